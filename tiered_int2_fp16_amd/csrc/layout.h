// Physical layouts of bf16 windows and b-bit (2, 4, 8) ledger entries.
//
// Both are built around one wave64 matrix-core operand shape (16x16x32 MFMA on
// gfx950): lane l of a wave holds 8 consecutive values of row l%16 at column
// block l/16.  Every per-lane 16-byte chunk of a 32-token tile is stored where
// a linear wave load (lane l reads chunk l) drops it straight into the operand
// register that needs it - no shuffles, no LDS transposes.
//
// Token order inside a 32-token tile.  Row m (0..15) of the QK product's block
// blk (0, 1) is token qk_token(blk, m) = 8*(m/4) + 4*blk + m%4.  With that
// choice the QK result a lane holds (rows 4*(l/16)+i of both blocks: tokens
// 8*(l/16) + 4*blk + i) is exactly the 8 tokens 8*(l/16)..+7 the PV product
// wants from that lane, so probabilities never move between lanes.  Tokens are
// otherwise in window order; the permutation only decides chunk placement.
//
// bf16 window block (per slot, per kv head): W/32 tiles of 64*D values, each
//   K part (32*D): chunk (cmb, lane), cmb = blk*(D/32) + kk, holds
//                  K[qk_token(blk, lane%16)][32*kk + 8*(lane/16) + e], e = 0..7
//   V part (32*D): chunk (nb, lane) holds V[8*(lane/16) + e][16*nb + lane%16]
// Ledger entry of b-bit codes (per slot, per kv head): W/32 tiles of
// 8*(b+1)*D bytes, each
//   Kc (4*b*D B) | Vc (4*b*D B) | Ks (2*D B) | Km (2*D B) | Vs (2*D B) | Vm (2*D B)
//   Kc, Vc: lane l owns b*D/16 bytes = b*D/64 little-endian 32-bit words; the
//   8 codes of a chunk go where one or two register operations turn a pair
//   of them into the two fp16 halves of a 32-bit register:
//   b = 2: word w carries the codes of chunks cmb = 2w (sel 0) and 2w+1
//     (sel 1); field f (bits 2f..2f+1) is element e = 2*(f%4) + f/8 of chunk
//     2w + (f/4)%2.  Fields (r + 4*sel, r + 4*sel + 8) sit 16 bits apart, so
//     one shift and one mask place a pair of codes in the two halves.
//   b = 4: word w is chunk w; field f (bits 4f..4f+3) is element
//     e = 2*(f%4) + f/4 (fields r and r + 4, 16 bits apart, are elements 2r
//     and 2r + 1).
//   b = 8: words 2c and 2c+1 are chunk c; byte e of that pair is element e
//     (a byte permute spreads elements 2r, 2r + 1 over the two halves).
//   Chunk numbering is that of the bf16 tile (K: cmb, V: nb).
//   Ks, Km: fp16 [D] scale / min of the tile's K group of each channel.
//   Vs, Vm: fp16 [D/32][32] scale / min of each token's V group j (channels
//     32j..32j+31), indexed [j][token].
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define KV_HD __host__ __device__ inline
#else
#define KV_HD inline
#endif

namespace kvtier {
namespace layout {

constexpr int kTileTokens = 32;

KV_HD int qk_token(int blk, int m) { return 8 * (m >> 2) + 4 * blk + (m & 3); }

// ---- bf16 tile: value offsets (in bf16 elements) within one 32-token tile
KV_HD int bf16_k_offset(int t, int d, int D) {
  const int blk = (t >> 2) & 1, m = 4 * (t >> 3) + (t & 3);
  const int cmb = blk * (D >> 5) + (d >> 5);
  const int lane = 16 * ((d >> 3) & 3) + m;
  return (cmb * 64 + lane) * 8 + (d & 7);
}
KV_HD int bf16_v_offset(int t, int d, int D) {
  const int lane = 16 * (t >> 3) + (d & 15);
  return 32 * D + ((d >> 4) * 64 + lane) * 8 + (t & 7);
}
// offset of (token t of the window, dim d) in a window block, K and V
KV_HD long bf16_window_k(int t, int d, int D) {
  return long(t >> 5) * 64 * D + bf16_k_offset(t & 31, d, D);
}
KV_HD long bf16_window_v(int t, int d, int D) {
  return long(t >> 5) * 64 * D + bf16_v_offset(t & 31, d, D);
}

// (token, dim) of element e of chunk (cmb, lane) of a tile's K part / V part
KV_HD void k_chunk_elem(int cmb, int lane, int e, int D, int* t, int* d) {
  const int kk_n = D >> 5;
  *t = qk_token(cmb / kk_n, lane & 15);
  *d = 32 * (cmb % kk_n) + 8 * (lane >> 4) + e;
}
KV_HD void v_chunk_elem(int nb, int lane, int e, int* t, int* d) {
  *t = 8 * (lane >> 4) + e;
  *d = 16 * nb + (lane & 15);
}
// element e of field f of a code word of chunk pair (2w, 2w+1)
KV_HD void field_elem(int w, int f, int* cmb, int* e) {
  *cmb = 2 * w + ((f >> 2) & 1);
  *e = 2 * (f & 3) + (f >> 3);
}

// element e of field f of code word w (b-bit codes): its chunk and element
KV_HD void field_elem_b(int bits, int w, int f, int* cmb, int* e) {
  if (bits == 2) {
    field_elem(w, f, cmb, e);
  } else if (bits == 4) {
    *cmb = w;
    *e = 2 * (f & 3) + (f >> 2);
  } else {
    *cmb = w >> 1;
    *e = 4 * (w & 1) + f;
  }
}

// ---- ledger tile: byte offsets within one 8*(b+1)*D-byte tile
struct LedgerTile {
  int kc, vc, ks, km, vs, vm, bytes;
  KV_HD LedgerTile(int D, int bits)
      : kc(0), vc(4 * bits * D), ks(8 * bits * D), km(8 * bits * D + 2 * D), vs(8 * bits * D + 4 * D),
        vm(8 * bits * D + 6 * D), bytes(8 * (bits + 1) * D) {}
};

// Code position of a chunk element: byte offset of its 32-bit word within the
// Kc (or Vc) area of the tile, and its bit position inside that word.
KV_HD void code_pos(int cmb, int lane, int e, int D, int bits, int* word_byte, int* bit) {
  const int lane_bytes = bits * D / 16;
  if (bits == 2) {
    const int w = cmb >> 1, sel = cmb & 1;
    const int f = (e >> 1) + 4 * sel + 8 * (e & 1);
    *word_byte = lane * lane_bytes + 4 * w;
    *bit = 2 * f;
  } else if (bits == 4) {
    *word_byte = lane * lane_bytes + 4 * cmb;
    *bit = 4 * ((e >> 1) + 4 * (e & 1));
  } else {
    *word_byte = lane * lane_bytes + 4 * (2 * cmb + (e >> 2));
    *bit = 8 * (e & 3);
  }
}
// K code of (token t of the tile, dim d)
KV_HD void k_code_pos(int t, int d, int D, int bits, int* word_byte, int* bit) {
  const int blk = (t >> 2) & 1, m = 4 * (t >> 3) + (t & 3);
  code_pos(blk * (D >> 5) + (d >> 5), 16 * ((d >> 3) & 3) + m, d & 7, D, bits, word_byte, bit);
}
// V code of (token t of the tile, dim d)
KV_HD void v_code_pos(int t, int d, int D, int bits, int* word_byte, int* bit) {
  code_pos(d >> 4, 16 * (t >> 3) + (d & 15), t & 7, D, bits, word_byte, bit);
}

}  // namespace layout
}  // namespace kvtier
