// svdq_layout.h -- byte layout of the packed layer blob and of the forward
// workspace.  Shared by the host pack and the device launch code of the
// library (not by any checker).
//
// Every 4-bit operand is stored as matrix-core fragments: a wave loads a
// whole fragment with one 16-byte load per lane.  Rows are output columns n
// for the weight and tokens m for the activations.
//   MXFP4 (32 x 32 x 64 scaled MFMA): per 32-row tile and 128-deep K step,
//          2 halves x 64 lanes x 16 bytes; in half h, lane l holds row l % 32
//          and the 32 E2M1 codes of k in [64h + 32(l / 32), +32) of the step
//          (element 2i in the low nibble of byte i) -- one e8m0 block.
//   INT4 (16 x 16 x 64 integer MFMA): per 16-row tile and step, 64 lanes x
//          16 bytes; lane l holds row l % 16 and, in bytes [4c, 4c+4), the
//          8 codes of k in [32c + 8q, 32c + 8q + 8), q = l / 16: bytes
//          [0, 8) belong to the step's first 64-group, [8, 16) to the
//          second.  (The order of k inside a group is free for an integer
//          dot product; this one lets the activation kernel write each
//          lane's 16 bytes straight from coalesced loads of X.)
//   INT8 (32 x 32 x 32 integer MFMA): per 32-row tile and 64-deep K step,
//          2 halves x 64 lanes x 16 bytes; in half h, lane l holds row l % 32
//          and the int8 codes of k in [32h + 16(l / 32), +16) of the step --
//          the same 2 KB per tile and step as an MXFP4 128-deep step.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace svdq {

constexpr int KSTEP = 128;         // K covered by one fragment step
constexpr int FRAG_BYTES = 1024;   // 64 lanes x 16 bytes
constexpr int M_PAD = 256;         // workspace rows are padded to this
constexpr int HDR_BYTES = 256;
constexpr uint32_t BLOB_MAGIC = 0x51445653u;   // "SVDQ"
constexpr uint32_t BLOB_VERSION = 3u;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline int group_size(int fmt) { return fmt == 0 ? 64 : 32; }   // 4-bit formats
constexpr int FMT_INT8 = 2;                                       // whole-row scales
inline size_t code_bytes(int64_t rows, int64_t K, int fmt) {
  return fmt == FMT_INT8 ? size_t(rows) * size_t(K) : size_t(rows) * size_t(K) / 2;
}

// Header at the start of every blob (all later offsets are relative to the blob).
struct BlobHeader {
  uint32_t magic, version;
  int64_t K, N;
  int32_t rank, rank_active, rank_capacity, rank_slots, fmt, dtype, has_bias, pad0;
  uint64_t off_invlam, off_lam, off_l1x, off_l2, off_wq, off_sw, off_bias, total;
};
static_assert(sizeof(BlobHeader) <= HDR_BYTES, "header too large");

struct BlobOffsets {
  size_t invlam, lam, l1x, l2, wq, sw, bias, total;
};

// bytes of the weight scales
inline size_t weight_scale_bytes(int64_t K, int64_t N, int fmt) {
  if (fmt == FMT_INT8) return size_t(N) * 4;                                // INT8: fp32 per output channel
  if (fmt == 1) return size_t(N) * size_t(K / 32);                          // MX: one byte per 32-block
  return size_t(N / 16) * size_t(K / KSTEP) * 64;                           // INT4: 2 groups x 16 rows x fp16
}

inline BlobOffsets blob_offsets(int64_t K, int64_t N, int slots, int fmt) {
  BlobOffsets o;
  size_t p = HDR_BYTES;
  o.invlam = p; p = align256(p + size_t(K) * 4);
  o.lam = p;    p = align256(p + size_t(K) * 4);
  o.l1x = p;    p = align256(p + size_t(K) * slots * 2);
  o.l2 = p;     p = align256(p + size_t(slots) * N * 2);
  o.wq = p;     p = align256(p + code_bytes(N, K, fmt));
  o.sw = p;     p = align256(p + weight_scale_bytes(K, N, fmt));
  o.bias = p;   p = align256(p + size_t(N) * 4);
  o.total = p;
  return o;
}

struct WsOffsets {
  int64_t Mp;
  size_t xq, sx, t, total;
};

inline size_t act_scale_bytes(int64_t Mp, int64_t K, int fmt) {
  if (fmt == FMT_INT8) return size_t(Mp) * 4;                               // fp32 per token
  if (fmt == 1) return size_t(Mp) * size_t(K / 32);
  return size_t(Mp / 16) * size_t(K / KSTEP) * 64;
}

inline WsOffsets ws_offsets(int64_t M, int64_t K, int slots, int fmt) {
  WsOffsets w;
  w.Mp = round_up(M > 0 ? M : 1, M_PAD);
  size_t p = 0;
  w.xq = p; p = align256(p + code_bytes(w.Mp, K, fmt));
  w.sx = p; p = align256(p + act_scale_bytes(w.Mp, K, fmt));
  w.t = p;  p = align256(p + size_t(w.Mp) * slots * 2);
  w.total = p;
  return w;
}

// ---- element -> position maps (used by the host pack and the exporters) ----

// Code of (row r, k) in a fragment array with K columns: byte offset and
// nibble (0 = low) within it (INT8: the whole byte, nib = 0).
inline void code_pos(int64_t r, int64_t k, int64_t K, int fmt, size_t* byte, int* nib) {
  const int64_t nsteps = K / KSTEP, s = k / KSTEP, kk = k % KSTEP;
  if (fmt == FMT_INT8) {
    const int64_t t = r / 32, s64 = k / 64, h = (k % 64) / 32, k32 = k % 32;
    const int64_t lane = (r % 32) + 32 * (k32 / 16);
    *byte = size_t((((t * (K / 64) + s64) * 2 + h) * 64 + lane) * 16 + k32 % 16);
    *nib = 0;
  } else if (fmt == 1) {
    int64_t t = r / 32, b = kk / 32, c = kk % 32, h = b / 2;
    int64_t lane = (r % 32) + 32 * (b % 2);
    *byte = size_t(((t * nsteps + s) * 2 + h) * 1024 + lane * 16 + c / 2);
    *nib = int(c % 2);
  } else {
    int64_t t = r / 16, c = kk / 32, q = (kk % 32) / 8, e = kk % 8;
    int64_t lane = (r % 16) + 16 * q;
    *byte = size_t(((t * nsteps + s) * 64 + lane) * 16 + 4 * c + e / 2);
    *nib = int(e % 2);
  }
}

// MX e8m0 scale of (row r, 32-block b): byte offset.  Per (pair of 32-row
// tiles, step): 64 lanes x 4 bytes; lane l holds the scales of its fragment
// row and K block in both halves of both tiles, byte 2 (tile % 2) + half
// (the scaled MFMA picks it with op_sel).
inline size_t mx_scale_pos(int64_t r, int64_t b, int64_t K) {
  int64_t t = r / 32, s = b / 4, bb = b % 4, h = bb / 2;
  int64_t lane = (r % 32) + 32 * (bb % 2);
  return size_t((((t / 2) * (K / KSTEP) + s) * 64 + lane) * 4 + 2 * (t % 2) + h);
}

// INT4 fp16 scale of weight (column n, 64-group G): element (uint16) offset.
// Per (16-column tile, step): [n % 16][group in step], so one dword holds a
// column's two scales of the step, low half first (the GEMM's scale MFMA
// takes that dword as its k = 0, 1 operand).
inline size_t int4_wscale_pos(int64_t n, int64_t G, int64_t K) {
  int64_t t = n / 16, s = G / 2, g = G % 2;
  return size_t(((t * (K / KSTEP) + s) * 16 + n % 16) * 2 + g);
}

// INT4 fp16 scale of activation (token m, 64-group G): element offset.
// Per (16-token tile, step): [m % 16][group in step].
inline size_t int4_xscale_pos(int64_t m, int64_t G, int64_t K) {
  int64_t t = m / 16, s = G / 2, g = G % 2;
  return size_t(((t * (K / KSTEP) + s) * 16 + (m % 16)) * 2 + g);
}

// 16-bit low-rank operand of the GEMM epilogue: (row r, rank j), rows are
// n for L2 and m for T.
//   MXFP4 and INT8 (32 x 32 x 16 MFMA): per (32-row tile, 16-rank chunk) 64 lanes x 8;
//          lane l holds row l % 32 and j in [16c + 8(l / 32), +8).
//   INT4 (16 x 16 x 32 MFMA): per (16-row tile, 32-rank chunk) 64 lanes x 8;
//          lane l holds row l % 16 and j in [32c + 8(l / 16), +8).
inline size_t lr_pos(int64_t r, int64_t j, int slots, int fmt) {
  if (fmt == 1 || fmt == FMT_INT8) {
    int64_t t = r / 32, c = j / 16, jj = j % 16;
    int64_t lane = (r % 32) + 32 * (jj / 8);
    return size_t(((t * (slots / 16) + c) * 64 + lane) * 8 + jj % 8);
  }
  int64_t t = r / 16, c = j / 32, jj = j % 32, q = jj / 8, e = jj % 8;
  int64_t lane = (r % 16) + 16 * q;
  return size_t(((t * (slots / 32) + c) * 64 + lane) * 8 + e);
}

// 16-bit L1x as the activation kernel reads it: (k, rank j).
// Per (128-step, 16-rank tile, MFMA c = 0..3): 64 lanes x 8; lane covers
// rank (j % 16) and 8 consecutive k of the step, the A operand of a
// 16 x 16 x 32 MFMA whose B operand is the same lane's slice of X:
//   INT4:  k in [32c + 8g, +8), g = lane / 16 (a lane holds a quarter of
//          every 32-block of the step);
//   MXFP4: k in [32g + 8c, +8) (lane group g holds the whole 32-block g).
inline size_t l1x_pos(int64_t k, int64_t j, int slots, int fmt) {
  const int64_t s = k / KSTEP, kk = k % KSTEP, e = kk % 8, jt = j / 16;
  const int64_t c = fmt == 1 ? (kk % 32) / 8 : kk / 32;
  const int64_t g = fmt == 1 ? kk / 32 : (kk % 32) / 8;
  const int64_t lane = (j % 16) + 16 * g;
  return size_t((((s * (slots / 16) + jt) * 4 + c) * 64 + lane) * 8 + e);
}

}  // namespace svdq
