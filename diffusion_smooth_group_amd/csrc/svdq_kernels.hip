// svdq_kernels.hip -- gfx950 (MI355X) kernels of the SVDQuant linear and the
// forward entry points of the C ABI (include/svdq.h).
//
// SVDQuant paper ("SVDQuant: Absorbing Outliers by Low-Rank Components for
// 4-Bit Diffusion Models"): the forward is Eq. 5 of §4.2, fused the way §4.3
// (Fig. 6b) describes -- the low-rank down-projection shares its input with
// the activation quantizer, the up-projection shares its output with the
// 4-bit product -- so the 16-bit branch adds no extra pass over X or Y.
//
//   k1_act   one pass over X: per-channel 1/lambda, group absmax (in
//            registers / one lane exchange), 4-bit codes and scales written
//            straight into matrix-core fragment order, and T = X L1x on
//            bf16/f16 MFMA from the same registers.
//   k2_gemm  4-bit GEMM on MFMA: MXFP4 on V_MFMA_SCALE_F32_16X16X128_F8F6F4
//            with the e8m0 block scales applied by the matrix core; INT4 on
//            V_MFMA_I32_16X16X64_I8 (nibbles widened to 16*q int8), exact
//            int32 per-group products dequantized in fp32.  The epilogue adds
//            T L2 on bf16/f16 MFMA into the same accumulators, then bias,
//            optional GELU, rounding and the store.
//
// Operand orientation: the weight fragment is the MFMA "A" operand (rows =
// output columns n), the activation fragment is "B" (columns = tokens m), so
// each lane ends with 4 consecutive n of one token and stores 8 bytes.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>
#include <mutex>
#include <atomic>
#include <vector>

#include "svdq.h"
#include "svdq_layout.h"

namespace svdq {
svdq_status validate_layer(const svdq_layer* L);
}

namespace {

using svdq::KSTEP;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int MAXJT = SVDQ_MAX_RANK_CAPACITY / 16;   // 16-rank tiles of T

// ------------------------------------------------------------ number formats
template <int DT>
__device__ __forceinline__ float h2f(unsigned v) {
  if constexpr (DT == SVDQ_BF16) return __uint_as_float(v << 16);
  else return float(__builtin_bit_cast(_Float16, (unsigned short)v));
}

template <int DT>
__device__ __forceinline__ unsigned f2h(float f) {   // round to nearest even
  if constexpr (DT == SVDQ_BF16) {
    unsigned u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  } else {
    return (unsigned)__builtin_bit_cast(unsigned short, (_Float16)f);
  }
}

// two floats -> two 16-bit values (round to nearest even) in one dword, low
// half first; one v_cvt_pk_{bf16,f16}_f32 on this target
template <int DT>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  if constexpr (DT == SVDQ_BF16) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, bf16x2_t{(__bf16)a, (__bf16)b});
  } else {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, f16x2_t{(_Float16)a, (_Float16)b});
  }
}

template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == SVDQ_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// s_waitcnt vmcnt(n) leaving expcnt and lgkmcnt unconstrained
#define SVDQ_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8))
// s_waitcnt lgkmcnt(0) leaving vmcnt and expcnt unconstrained
#define SVDQ_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (0x7 << 4))

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Max of a non-negative float over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four
// lanes q = 0..3 of one token in the activation kernel).  permlane16_swap
// with both operands x leaves x of lanes l and l ^ 16 in its two results,
// permlane32_swap likewise for l ^ 32; non-negative floats order as their
// bit patterns.
__device__ __forceinline__ unsigned umax_u(unsigned a, unsigned b) { return a > b ? a : b; }
__device__ __forceinline__ float quad_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned m16 = umax_u(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(m16, m16, false, false);
  return __uint_as_float(umax_u(r32[0], r32[1]));
}

// e8m0 exponent of an MXFP4 block with absmax a: the biased exponent of
// t = fl32(a / 6) plus one if t is not a power of two (so 2^(e-127) >= t),
// 0 for t = 0, at most 254.  For a normal a = 1.f x 2^(B-127) with B >= 3,
// a / 6 = (1.f / 1.5) 2^(B-129) never rounds across a power of two, and t is
// itself a power of two only when 1.f = 1.5, so e = B - 2 + (f > 0.5)
// exactly; tiny a (B < 3, t possibly subnormal) takes the division.
__device__ __forceinline__ int e8m0_fast(float a) {      // exact for a >= 2^-124
  const unsigned b = __float_as_uint(a);
  const int B = int(b >> 23);                    // a >= 0: no sign bit
  return B >= 255 ? 254 : B - 2 + ((b & 0x7FFFFFu) > 0x400000u ? 1 : 0);
}
__device__ __forceinline__ int e8m0_slow(float a) {      // any a >= 0
  const float t = a / 6.0f;
  const unsigned tb = __float_as_uint(t);
  if (t == 0.0f) return 0;
  const int e = int(tb >> 23) + ((tb & 0x7FFFFFu) != 0u ? 1 : 0);
  return e > 254 ? 254 : e;
}
__device__ __forceinline__ bool e8m0_needs_slow(float a) { return (__float_as_uint(a) >> 23) < 3u; }

// INT4 group quantization of one 128-deep K step of 16 tokens, in the
// activation fragment layout: lane l = m + 16q holds token m and, in chunk
// c = 0..3, the smoothed values xh[c][0..7] of k in [32c + 8q, +8), with am[c]
// their maximum magnitude; a 64-group is chunks 2g, 2g + 1 of the token's
// four lanes, whose maxima meet through quad_max.  Writes the lane's 16 code
// bytes (element order of the fragment: chunk c in bytes [4c, 4c + 4)) and
// the fp16 scale bits of the two groups.  The activation kernel and the
// chained GEMM epilogue both quantize through this function.
__device__ __forceinline__ void int4_quant_step(const float (&xh)[4][8], const float (&am)[4], unsigned (&d)[4],
                                                unsigned (&sh)[2]) {
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float a = quad_max(fmaxf(am[2 * g], am[2 * g + 1]));
    const float sc = fminf(a / 7.0f, 65504.0f);
    sh[g] = f2h<SVDQ_F16>(sc);
    const float s32 = h2f<SVDQ_F16>(sh[g]);
    // The code is rint(fl(x / s)).  x * fl(1/s) is within 1.5 ulp of
    // fl(x / s), below 2^-19 wherever |x / s| < 10.5 (larger values
    // clamp to 7 either way), so the two roundings can only differ when
    // it lies within 2^-18 of a half-integer; such lanes redo the group
    // with the correctly rounded division.
    const float inv = s32 != 0.0f ? 1.0f / s32 : 0.0f;
    unsigned near = 0u;                 // bit 8 cc + e: element (cc, e) lies near a half-integer
    float r[2][8];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = xh[2 * g + cc][e] * inv;
        r[cc][e] = rintf(qv);
        near |= (fabsf(qv - r[cc][e]) >= 0.5f - 0x1p-18f ? 1u : 0u) << (8 * cc + e);
      }
    if (__builtin_expect(near != 0u, 0)) {
      // only the near elements take the division (each one under a branch
      // the wave skips when no lane needs it)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (near & (1u << (8 * cc + e))) r[cc][e] = s32 != 0.0f ? rintf(xh[2 * g + cc][e] / s32) : 0.0f;
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      unsigned v = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float rc = __builtin_amdgcn_fmed3f(r[cc][e], -7.0f, 7.0f);   // clamp, one v_med3_f32
        v |= (unsigned(int(rc)) & 0xFu) << (4 * e);
      }
      d[2 * g + cc] = v;
    }
  }
}

// ------------------------------------------------------------------- k1_act
struct K1Params {
  const uint16_t* X;
  int64_t ldx, M, K;
  const float* invlam;
  const uint16_t* l1x;   // tiled for this kernel
  int slots, njt;
  uint8_t* xq;
  uint8_t* sx;
  uint16_t* t;
};

// One workgroup = 16 tokens (TT = 2: two 16-token tiles, each wave taking
// its steps for both, so a step's L1x fragments -- the down-projection's A
// operands, twice the step's X bytes at rank 32 -- are loaded once for 32
// tokens; one wave per SIMD); its 4 waves take the 128-deep K steps round
// robin, and lane l = m + 16q holds token m.  MXFP4: lane group q holds the
// whole 32-block q of a step (k in [32q + 8c, +8) for c = 0..3), so the
// block maximum, exponent and codes are the lane's own work.  INT4: in
// chunk c = 0..3 of a step the lane holds k in [32c + 8q, 32c + 8q + 8), so
// a 64-group is chunks 2g and 2g + 1 of the token's four lanes.
//
// Loads.  MXFP4, and INT4 up to rank 32, read X row-contiguously: load c of
// a step brings rows 4c .. 4c + 3 of the tile, 16 lanes per 256-byte row
// segment, so every load instruction covers whole cache lines (the lane map
// above touches 32 lines per instruction, a quarter of each, and streams X
// markedly slower).  Each step then passes through the wave's own 4 KB LDS
// buffer into the lane map: a lane stores its piece at its position in the
// row and reads its own pieces back.  Lane (row r, position i) loads piece
// i ^ r of the row, so a piece P of row m sits at position P ^ m and the
// lane-map reads of 16 consecutive lanes fall in distinct banks.  INT4 with
// wider ranks loads in the lane map itself: the extra offset registers would
// spill beside its L1x fragments.
//
// Latency.  The vector memory counter retires in issue order, so waiting for
// a short (L2) load also waits for every older HBM load.  Each step is
// quantized and then projected (the down-projection MFMAs from the X still
// in registers run on the matrix unit under the next step's quantization).
// A wave keeps a rolling ring of steps in flight (step i + R - 1's L1x and X
// requested before step i is processed), so with one workgroup per compute
// unit its quantization runs under its own stream.  When more than two
// workgroups per compute unit queue up (CHUNK), MXFP4 instead requests
// a whole chunk of steps' X at once: the resident workgroups' compute then
// covers each other's waits, and the deeper request streams faster.  Every
// memory operation is unconditional (indices past the wave's last step are
// clamped, so padding steps rewrite identical codes; their MFMAs are
// skipped), which keeps the compiler's counter bookkeeping exact.
// invlambda is copied to LDS (when it fits) through registers.  Codes,
// scales and T leave with non-temporal stores: the GEMM that reads them runs
// on every XCD and reads them from memory anyway, and lines that do not sit
// dirty in this kernel's L2s need no write-back before the GEMM may start.
constexpr int K1_IL_LDS_MAX_K = 16384;
constexpr int K1_XBUF_BYTES = 4 * 4096;    // the four waves' step buffers
template <int NJT> struct K1Ring { static constexpr int value = NJT <= 2 ? 3 : (NJT <= 4 ? 2 : 1); };
template <int NJT> struct K1Chunk { static constexpr int value = NJT <= 2 ? 6 : 2; };
template <int NJT> struct K1LRing { static constexpr int value = NJT <= 4 ? 2 : 1; };

// QUANT = false runs the down-projection alone (the unfused low-rank
// baseline's separate pass over X): no codes, scales or invlambda.
template <int FMT, int DT, int NJT, bool IL_LDS, bool QUANT = true, bool CHUNK = false, int TT = 1>
__global__ __launch_bounds__(256, TT == 1 ? 2 : 1) void k1_act(K1Params p) {   // TT = 1: two waves per SIMD at least
  // one LDS object: invlambda[0, K) (if IL_LDS), then the T reduction
  // buffer, then the waves' step buffers
  extern __shared__ __attribute__((aligned(16))) uint8_t k1_lds[];
  constexpr bool MXC = CHUNK && FMT == SVDQ_FMT_MXFP4_G32 && NJT <= 4;   // chunked requests
  constexpr int R = MXC ? K1Chunk<NJT>::value : K1Ring<NJT>::value;   // X slots per wave
  constexpr int LR = MXC ? K1LRing<NJT>::value : R;                    // L1x slots per wave
  static_assert(TT == 1 || !MXC, "two-tile workgroups take the rolling ring");
  const int mt0 = int(blockIdx.x) * TT;          // first 16-token tile of this workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  // Rows past M (the workspace's padding up to its 256-row multiple) repeat
  // row M - 1: their codes, scales and T only ever meet GEMM outputs that are
  // not stored, and every load stays unconditional.
  const int nsteps = int(p.K / KSTEP);
  const int nmine = (nsteps - wave + 3) / 4;     // this wave's steps: wave, wave + 4, ...
  // MXFP4: lane group q holds the whole 32-block q of each step (k in
  // [32q + 8c, +8) for load c); INT4: a quarter of every block (k in
  // [32c + 8q, +8)), so a 64-group spans the four lanes of a token.
  constexpr bool MXL = FMT == SVDQ_FMT_MXFP4_G32;
  constexpr bool XT = MXL || NJT <= 2;           // row-contiguous loads through LDS
  // XT: load c's row (4c + lane / 16) and the piece this lane loads,
  // (lane % 16) ^ row, as element offsets from the tile's first row (a row
  // past M reads row M - 1, which may lie before the tile).  Otherwise the
  // lane-map row and its k offset.
  // (the offsets of every tile of the workgroup count from its first tile's row)
  const uint16_t* xtile = p.X + int64_t(mt0) * 16 * p.ldx;
  int xo[TT][XT ? 4 : 1];
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    if constexpr (XT) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 4 * c + (lane >> 4);
        xo[u][c] = int(min(int64_t(mt0 + u) * 16 + r, p.M - 1) - int64_t(mt0) * 16) * int(p.ldx) + 8 * ((lane & 15) ^ r);
      }
    } else {
      xo[u][0] = int(min(int64_t(mt0 + u) * 16 + m, p.M - 1) - int64_t(mt0) * 16) * int(p.ldx) + 8 * q;
    }
  }
  const float* il_lds = reinterpret_cast<const float*>(k1_lds);
  // invlambda is copied in whole 1 KB pieces, so its LDS copy spans K rounded up to 256
  const size_t il_span = IL_LDS ? size_t((p.K + 255) & ~int64_t(255)) * 4 : 0;
  f32x4* red = reinterpret_cast<f32x4*>(k1_lds + il_span);   // [4][TT][NJT][64]
  uint8_t* xb = k1_lds + il_span + size_t(4) * TT * NJT * 64 * 16 + wave * 4096 * TT;   // this wave's step buffers

  // invlambda goes to LDS through registers and LDS stores, not direct
  // global->LDS loads: after those the compiler makes the first LDS read
  // wait for every outstanding load (all of the chunk's X).  Up to
  // K = 4096 each thread holds its pieces while the chunk's X is requested
  // and stores them afterwards; larger K copies first.
  constexpr int ILR = 4;
  const bool il_regs = p.K <= ILR * 1024;         // uniform
  f32x4 ilv[ILR];
  auto il_store = [&]() {
#pragma unroll
    for (int i = 0; i < ILR; ++i) {
      const int pc = int(threadIdx.x) + 256 * i;
      if (pc * 4 < p.K) *reinterpret_cast<f32x4*>(k1_lds + pc * 16) = ilv[i];
    }
    SVDQ_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
  };
  if constexpr (IL_LDS) {
    if (il_regs) {
      // unconditional loads (an index past K/4 re-reads the last piece, which
      // il_store does not store)
      const int last = int(p.K / 4) - 1;
#pragma unroll
      for (int i = 0; i < ILR; ++i) {
        const int pc = min(int(threadIdx.x) + 256 * i, last);
        ilv[i] = *reinterpret_cast<const f32x4*>(p.invlam + pc * 4);
      }
    } else {
      for (int pc = int(threadIdx.x); pc * 4 < p.K; pc += 256)
        *reinterpret_cast<f32x4*>(k1_lds + pc * 16) = *reinterpret_cast<const f32x4*>(p.invlam + pc * 4);
      SVDQ_WAIT_LGKM0();
      __builtin_amdgcn_s_barrier();
    }
  }

  f32x4 tacc[TT][NJT > 0 ? NJT : 1];
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int j = 0; j < NJT; ++j) tacc[u][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int njc = p.njt > 0 ? p.njt - 1 : 0;
  // the step of ring index i: clamped to the wave's last step, and step 0
  // for a wave without steps (K < 512), whose ring prologue still loads
  auto step_of = [&](int i) { return nmine > 0 ? wave + 4 * (i < nmine ? i : nmine - 1) : 0; };
  u32x4 xr[R][TT][4];
  u32x4 lring[LR][NJT > 0 ? NJT : 1][4];
  auto load_x = [&](int slot, int i) {
    const int s = step_of(i);
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (XT) xr[slot][u][c] = *reinterpret_cast<const u32x4*>(xtile + (xo[u][c] + s * KSTEP));
        else xr[slot][u][c] = *reinterpret_cast<const u32x4*>(xtile + (xo[u][0] + s * KSTEP + 32 * c));
      }
  };
  // a landed step through the wave's LDS buffer into the lane map: row r at
  // r * 256, each lane's piece at its own position; piece P of row m is read
  // back from position P ^ m.  The wave's LDS operations run in order, so
  // the next step's stores cannot overtake these reads.
  auto to_lane_map = [&](int slot) {
    if constexpr (!XT) return;
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4*>(xb + u * 4096 + (4 * c + (lane >> 4)) * 256 + 16 * (lane & 15)) = xr[slot][u][c];
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int P = MXL ? 4 * q + c : 4 * c + q;
        xr[slot][u][c] = *reinterpret_cast<const u32x4*>(xb + u * 4096 + m * 256 + 16 * (P ^ m));
      }
  };
  auto load_l1x = [&](int slot, int i) {
    const int s = step_of(i);
    const u32x4* l1 = reinterpret_cast<const u32x4*>(p.l1x) + (size_t(s) * (p.slots / 16)) * 4 * 64 + lane;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
      for (int c = 0; c < 4; ++c) lring[slot][jt][c] = l1[((jt < njc ? jt : njc) * 4 + c) * 64];
  };

  // quantize one step: codes and scales of the 16 tokens of tile mt x 128 k
  auto quantize = [&](const u32x4 (&xq)[4], int s, int mt) {
    // smoothed values x_hat = x * invlambda (one fp32 multiply)
    float xh[4][8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = s * KSTEP + (MXL ? 32 * q + 8 * c : 32 * c + 8 * q);
      f32x4 il0, il1;
      if constexpr (IL_LDS) {
        il0 = *reinterpret_cast<const f32x4*>(il_lds + k);
        il1 = *reinterpret_cast<const f32x4*>(il_lds + k + 4);
      } else {
        il0 = *reinterpret_cast<const f32x4*>(p.invlam + k);
        il1 = *reinterpret_cast<const f32x4*>(p.invlam + k + 4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned w = xq[c][e];
        const f32x4& il = e < 2 ? il0 : il1;
        xh[c][2 * e] = h2f<DT>(w & 0xFFFFu) * il[(2 * e) & 3];
        xh[c][2 * e + 1] = h2f<DT>(w >> 16) * il[(2 * e + 1) & 3];
      }
    }
    float am[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      am[c] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am[c] = fmaxf(am[c], fabsf(xh[c][e]));
    }

    if constexpr (FMT == SVDQ_FMT_INT4_G64) {
      unsigned d[4];
      unsigned sh[2];
      int4_quant_step(xh, am, d, sh);
      uint8_t* frag = p.xq + (size_t(mt) * nsteps + s) * svdq::FRAG_BYTES;
      __builtin_nontemporal_store(u32x4{d[0], d[1], d[2], d[3]}, reinterpret_cast<u32x4*>(frag + lane * 16));
      if (q == 0)
        __builtin_nontemporal_store(sh[0] | (sh[1] << 16), reinterpret_cast<unsigned*>(p.sx) + (size_t(mt) * nsteps + s) * 16 + m);
    } else {
      // the lane's own block: maximum, e8m0 exponent, 32 codes
      float a = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) a = fmaxf(a, am[c]);
      int ex = e8m0_fast(a);
      float scl = __uint_as_float(unsigned(ex) << 23);
      if (__builtin_expect(e8m0_needs_slow(a), 0)) {
        ex = e8m0_slow(a);
        scl = ex != 0 ? __uint_as_float(unsigned(ex) << 23) : 1.0f;   // an all-zero block uses scale 1
      }
      // The packed fp32 -> E2M1 conversion divides by the power-of-two scale
      // 2^(e-127) (exact) and rounds to the nearest E2M1 value, ties to the
      // even mantissa, saturating at 6, keeping the sign of zero -- the group
      // quantizer's rule.  Each call writes its two codes into the selected
      // byte of the dword.
      unsigned d[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        unsigned v = 0u;
        v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, xh[c][0], xh[c][1], scl, 0);
        v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, xh[c][2], xh[c][3], scl, 1);
        v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, xh[c][4], xh[c][5], scl, 2);
        v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, xh[c][6], xh[c][7], scl, 3);
        d[c] = v;
      }
      // 32-row fragment tile t32 = mt / 2; block q of the step -> half q / 2,
      // lane (row in the 32-tile) + 32 (q % 2): one whole 16-byte piece
      const int t32 = mt >> 1, r32 = 16 * (mt & 1) + m;
      __builtin_nontemporal_store(u32x4{d[0], d[1], d[2], d[3]},
          reinterpret_cast<u32x4*>(p.xq + ((size_t(t32) * nsteps + s) * 2 + (q >> 1)) * 1024 + (r32 + 32 * (q & 1)) * 16));
      // scale byte 2 (t32 % 2) + q / 2 of the dword of lane (row + 32 (q % 2))
      __builtin_nontemporal_store(uint8_t(ex), p.sx + ((size_t(t32 >> 1) * nsteps + s) * 64 + r32 + 32 * (q & 1)) * 4 + 2 * (t32 & 1) + (q >> 1));
    }
  };

  // one step: quantize, then its share of the down-projection
  // T^T += L1x^T X^T on the raw 16-bit inputs (the matrix unit runs it under
  // the next step's quantization); a padding step past the wave's last (its
  // index clamped, so it rewrites identical codes) adds nothing
  auto project = [&](int slot, int lslot, int i) {
    if (i < nmine) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int u = 0; u < TT; ++u) tacc[u][jt] = mfma16<DT>(lring[lslot][jt][c], xr[slot][u][c], tacc[u][jt]);
    }
  };
  if constexpr (MXC) {
    // chunks of R steps: the L1x of the first LR steps, then all of the
    // chunk's X; the steps are taken as they land, L1x streamed LR ahead
    for (int i0 = 0; i0 < nmine; i0 += R) {
#pragma unroll
      for (int r = 0; r < LR; ++r) load_l1x(r, i0 + r);
#pragma unroll
      for (int d = 0; d < R; ++d) load_x(d, i0 + d);
      if constexpr (IL_LDS) {
        // the invlambda pieces were requested before this chunk's X
        if (i0 == 0 && il_regs) il_store();
      }
#pragma unroll
      for (int d = 0; d < R; ++d) {
        to_lane_map(d);
        if constexpr (QUANT) {
          // (each tile's ring slot named at the call: a slot index passed
          // through another lambda cost the one-tile kernels registers)
#pragma unroll
          for (int u = 0; u < TT; ++u) quantize(xr[d][u], step_of(i0 + d), mt0 + u);
        }
        project(d, d % LR, i0 + d);
        if (d + LR < R) load_l1x(d % LR, i0 + d + LR);
      }
    }
    if constexpr (IL_LDS) {
      // a wave without K steps (K < 512) still stores its invlambda pieces
      // and meets the barrier, so the barriers pair up across waves
      if (nmine <= 0 && il_regs) il_store();
    }
  } else {
    // rolling ring of R steps: step i + R - 1 is requested (L1x first, then
    // X) before step i is quantized and projected, so each wave keeps R
    // steps in flight and its first steps return while later ones stream
    // (with R = 1 the wide L1x of a large rank is requested after the
    // quantization so it is not live across it)
    auto load_step = [&](int slot, int i) {
      if constexpr (R > 1) load_l1x(slot, i);
      load_x(slot, i);
    };
#pragma unroll
    for (int r = 0; r + 1 < R; ++r) load_step(r, r);
    if constexpr (IL_LDS) {
      // every wave stores its invlambda pieces (requested before any X) and
      // meets this barrier, K steps or not
      if (il_regs) il_store();
    }
    for (int i0 = 0; i0 < nmine; i0 += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) {
        load_step((d + R - 1) % R, i0 + d + R - 1);
        to_lane_map(d);
        if constexpr (QUANT) {
          // (each tile's ring slot named at the call: a slot index passed
          // through another lambda cost the one-tile kernels registers)
#pragma unroll
          for (int u = 0; u < TT; ++u) quantize(xr[d][u], step_of(i0 + d), mt0 + u);
        }
        if constexpr (R == 1) load_l1x(d, i0 + d);
        project(d, d, i0 + d);
      }
    }
  }

  if constexpr (NJT > 0) {
    // T = the four waves' partial sums (fixed order), rounded once to 16 bits
    if (p.njt == 0) return;
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) red[((wave * TT + u) * NJT + jt) * 64 + lane] = tacc[u][jt];
    __syncthreads();
    for (int ij = wave; ij < TT * p.njt; ij += 4) {
      const int u = TT == 1 ? 0 : ij / p.njt, jt = TT == 1 ? ij : ij - u * p.njt, mt = mt0 + u;
      f32x4 v = red[(u * NJT + jt) * 64 + lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) v += red[((w * TT + u) * NJT + jt) * 64 + lane];
      // lane holds T[m][16 jt + 4q + i]; place it in the epilogue's B-fragment order
      const unsigned lo = pack2<DT>(v[0], v[1]);
      const unsigned hi = pack2<DT>(v[2], v[3]);
      uint16_t* dst;
      if constexpr (FMT == SVDQ_FMT_MXFP4_G32) {
        // 32-row tiles, 16-rank chunks: lane (row in tile) + 32 (j % 16 >= 8)
        const int t32 = mt >> 1, r32 = 16 * (mt & 1) + m;
        dst = p.t + ((size_t(t32) * (p.slots / 16) + jt) * 64 + r32 + 32 * (q >> 1)) * 8 + 4 * (q & 1);
      } else {
        // 16-row tiles, 32-rank chunks
        const int ldst = m + 16 * (2 * (jt & 1) + (q >> 1));
        dst = p.t + ((size_t(mt) * (p.slots / 32) + (jt >> 1)) * 64 + ldst) * 8 + 4 * (q & 1);
      }
      __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(dst));
    }
  }
}

// ------------------------------------------------------------------ k2_gemm
struct K2Params {
  const uint8_t* wq;
  const uint8_t* sw;
  const uint16_t* l2;
  const float* bias;
  const uint8_t* xq;
  const uint8_t* sx;
  const uint16_t* t;
  uint16_t* Y;
  int64_t ldy, M, N, K;
  int slots, nchunks, nchunks16;
  unsigned long long* trace;   // GEMM trace records (SVDQ_FLAG_TRACE) or null
  // Epilogue chaining of INT4 layers (k2_int4 with CHAIN): the next layer's
  // 1/lambda over this layer's N columns, its L1x (activation-kernel
  // tiling), its workspace codes and scales (written here), and fp32 partial
  // down-projections [N / 128][nx_Mp][nx_slots], one slab per 128-column tile
  const float* nx_invlam;
  const uint16_t* nx_l1x;
  uint8_t* nx_xq;
  uint8_t* nx_sx;
  float* nx_tp;
  int64_t nx_Mp;
  int nx_slots, nx_njt;
};

__device__ __forceinline__ i32x4 widen_nibbles(unsigned d0, unsigned d1) {
  // 16 signed nibbles -> 16 int8 holding 16*q (even elements first, then odd;
  // both operands use the same order, so the dot product is unchanged)
  return i32x4{int((d0 << 4) & 0xF0F0F0F0u), int((d1 << 4) & 0xF0F0F0F0u), int(d0 & 0xF0F0F0F0u),
               int(d1 & 0xF0F0F0F0u)};
}

// GEMM tracing (SVDQ_FLAG_TRACE): thread 0 of each workgroup writes the
// wall-clock counter and the shader-clock counter at the workgroup's start
// (records 0, 1) and, after a workgroup barrier, once every wave has issued
// its last store (records 2, 3).
constexpr int kTraceMax = 65536;       // workgroups a trace holds
__device__ __forceinline__ void trace_mark(unsigned long long* trace, int at) {
  const unsigned wg = blockIdx.x + gridDim.x * blockIdx.y;   // linear workgroup index (1-D and 2-D grids)
  if (at != 0 && trace != nullptr) __syncthreads();          // uniform: the whole workgroup takes it or none
  if (trace != nullptr && threadIdx.x == 0 && wg < unsigned(kTraceMax)) {
    const unsigned long long rt = __builtin_amdgcn_s_memrealtime(), ck = __builtin_amdgcn_s_memtime();
    trace[4 * size_t(wg) + at] = rt;
    trace[4 * size_t(wg) + at + 1] = ck;
  }
}

// GELU in its exact form x Phi(x), written without branches so an epilogue
// over many accumulators stays straight-line code.  With a = |x| and
// E(a) = erfc(a / sqrt2) / 2 (the Gaussian tail), GELU(x) = x - x E(a) for
// x >= 0 and x E(a) for x < 0, i.e. max(x, 0) - |x| E(a) in both cases (one
// fused multiply-add).  E(a) = 2^(-a^2 log2(e) / 2 + N(a)) where N, a
// degree-7 polynomial fitted to log2(erfcx(a / sqrt2) / 2) on [0, 4 sqrt2]
// (fit_gelu.py beside this file; a is clamped there), keeps the relative
// error of E, and of GELU, below 6e-6 in float32: one exp2 and ten other
// VALU instructions per element.  (Degree 6, at 3e-5, moves enough fp16
// roundings of an fc1 output that fc2's 4-bit codes of a few elements flip.)
__device__ __forceinline__ float gelu_erf(float x) {
  // clamp and max(x, 0) as v_med3_f32: fminf / fmaxf would first quiet
  // their inputs with an extra instruction each (a NaN x still yields NaN
  // through the last multiply-add)
  const float a = __builtin_amdgcn_fmed3f(fabsf(x), 0.0f, 5.656854249f);
  float p = -1.8169505645e-06f;
  p = __builtin_fmaf(p, a, 6.1296118065e-05f);
  p = __builtin_fmaf(p, a, -9.2855348124e-04f);
  p = __builtin_fmaf(p, a, 8.5016534895e-03f);
  p = __builtin_fmaf(p, a, -5.3950206273e-02f);
  p = __builtin_fmaf(p, a, 2.6287594084e-01f);
  p = __builtin_fmaf(p, a, -1.1512491604e+00f);
  p = __builtin_fmaf(p, a, -9.9999537112e-01f);
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(a * -0.72134752044f, a, p));   // E(a)
  return __builtin_fmaf(-fabsf(x), e, __builtin_amdgcn_fmed3f(x, 0.0f, 3.40282347e38f));   // max(x, 0)
}

// Epilogue chaining for INT4 layers (the next layer is INT4 too): the
// workgroup's staged 128 x 128 output tile -- the exact 16-bit bits this
// layer stores -- is one 128-deep K step of the next layer for 128 tokens.
// Wave w takes tokens 32w .. 32w + 31 in two 16-token sub-tiles with the
// activation kernel's INT4 lane layout (lane m + 16q holds k in
// [32c + 8q, +8) of chunk c): smoothing by the next layer's 1/lambda, codes
// and scales through int4_quant_step (so they are the activation kernel's
// bit for bit), and the down-projection over this step on the 16 x 16 x 32
// MFMA with the raw 16-bit values, written as fp32 to this column tile's
// slab (k_tfin sums the slabs in a fixed order).
template <int DT>
__device__ __forceinline__ void int4_chain_epilogue(const K2Params& p, const uint8_t* stage, int wave, int lane) {
  constexpr int OP = 64 * 2 + 16;                 // bytes per staged row (as in k2_int4)
  const int m = lane & 15, q = lane >> 4;
  const int s2 = blockIdx.x;                      // the next layer's K step: this tile's 128 columns
  const int nst2 = int(p.N / KSTEP);              // the next layer's K steps
  const int64_t mw0 = int64_t(blockIdx.y) * 128;
  const u32x4* l1 = reinterpret_cast<const u32x4*>(p.nx_l1x) + (size_t(s2) * (p.nx_slots / 16)) * 4 * 64 + lane;
  const int njc = p.nx_njt > 0 ? p.nx_njt - 1 : 0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = 32 * wave + 16 * u + m;         // token within the workgroup tile
    const int wm = t >> 6, row = t & 63;
    u32x4 xq[4];
    float xh[4][8], am[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int wn = c >> 1, col = 32 * (c & 1) + 8 * q;
      xq[c] = *reinterpret_cast<const u32x4*>(stage + (wn + 2 * wm) * (64 * OP) + row * OP + col * 2);
      const int k = s2 * KSTEP + 32 * c + 8 * q;
      const f32x4 il0 = *reinterpret_cast<const f32x4*>(p.nx_invlam + k);
      const f32x4 il1 = *reinterpret_cast<const f32x4*>(p.nx_invlam + k + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned w = xq[c][e];
        const f32x4& il = e < 2 ? il0 : il1;
        xh[c][2 * e] = h2f<DT>(w & 0xFFFFu) * il[(2 * e) & 3];
        xh[c][2 * e + 1] = h2f<DT>(w >> 16) * il[(2 * e + 1) & 3];
      }
      am[c] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am[c] = fmaxf(am[c], fabsf(xh[c][e]));
    }
    unsigned d[4], sh[2];
    int4_quant_step(xh, am, d, sh);
    const int64_t mt2 = (mw0 + 32 * wave + 16 * u) / 16;
    *reinterpret_cast<u32x4*>(p.nx_xq + (size_t(mt2) * nst2 + s2) * svdq::FRAG_BYTES + lane * 16) =
        u32x4{d[0], d[1], d[2], d[3]};
    if (q == 0) reinterpret_cast<unsigned*>(p.nx_sx)[(size_t(mt2) * nst2 + s2) * 16 + m] = sh[0] | (sh[1] << 16);
    // partial T[token][16 jt + 4q + i] over this step
    float* tp = p.nx_tp + (size_t(s2) * p.nx_Mp + size_t(mw0 + t)) * p.nx_slots + 4 * q;
    for (int jt = 0; jt < p.nx_njt; ++jt) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const int jj = jt < njc ? jt : njc;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma16<DT>(l1[(jj * 4 + c) * 64], xq[c], acc);
      *reinterpret_cast<f32x4*>(tp + 16 * jt) = acc;
    }
  }
}

// INT4 GEMM.  One workgroup = 128 output columns x 128 tokens; 4 waves in a
// 2 x 2 grid, each 64 x 64 (4 x 4 MFMA tiles of 16 x 16).  Per 64-group the
// integer MFMA gives the exact partial P_g (the nibbles are widened to
// 16 q per byte, so the MFMA sums 256 P_g); it is dequantized into fp32
// accumulators: acc += f32(256 P) * (s_w * s_x), and the epilogue takes the
// factor 2^-8 back out (exact: scaling by a power of two commutes with every
// rounding on the way).  The scale products come from the matrix core: a
// 16 x 16 x 16 fp16 MFMA whose operands hold only s_w (rows) and s_x
// (columns) at one k forms the 16 x 16 outer product in the accumulator
// layout of P, exactly (two fp16 values multiply exactly in fp32, the other
// terms are zero).  That leaves two VALU instructions per accumulator and
// group (convert, fused multiply-add).  The accumulators live in VGPRs,
// operands and scales are buffer loads with the lane's offset fixed and the
// step's offset in scalar registers (no per-step address arithmetic on the
// VALU), each step loaded one step ahead, and several waves share a SIMD.
template <int DT, bool GELU, bool CHAIN = false>
__global__ __launch_bounds__(256, 2) void k2_int4(K2Params p) {
  trace_mark(p.trace, 0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const bool k0 = lane < 16;             // lanes that carry k = 0..3 of a 16 x 16 x 16 operand
  // the scale operands' lane masks as AND masks (one instruction per
  // operand instead of a mask and a select): all bits on lanes 0..15, and
  // the low / high fp16 half of the scale dword for group 0 / 1
  const unsigned mk0 = k0 ? 0xFFFFFFFFu : 0u, mg0 = mk0 & 0x0000FFFFu, mg1 = mk0 & 0xFFFF0000u;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t n0 = int64_t(blockIdx.x) * 128 + wn * 64;
  const int64_t m0 = int64_t(blockIdx.y) * 128 + wm * 64;
  const int nt0 = int(n0 / 16), mt0 = int(m0 / 16);
  const int nsteps = int(p.K / KSTEP);

  // every span is below 2 GiB (checked on the host), so 32-bit offsets
  const __amdgpu_buffer_rsrc_t rwq = __builtin_amdgcn_make_buffer_rsrc((void*)p.wq, 0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rxq = __builtin_amdgcn_make_buffer_rsrc((void*)p.xq, 0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc((void*)p.sw, 0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc((void*)p.sx, 0, -1, 0x00020000);
  const int vcode = lane * 16;            // 16-byte fragment piece of this lane
  const int vsc = (lane & 15) * 4;        // this lane's column / token: both groups' fp16 scales

  // one step's raw operands: 4 weight and 4 token fragments (both 64-groups)
  // and the scale dwords (both groups) of the lane's weight column and token
  struct Ops {
    u32x4 a[4], b[4];
    unsigned sw[4], sx[4];
  };
  auto load = [&](Ops& o, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rwq, vcode, ((nt0 + i) * nsteps + s) * 1024, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) o.b[j] = __builtin_amdgcn_raw_buffer_load_b128(rxq, vcode, ((mt0 + j) * nsteps + s) * 1024, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) o.sw[i] = __builtin_amdgcn_raw_buffer_load_b32(rsw, vsc, ((nt0 + i) * nsteps + s) * 64, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) o.sx[j] = __builtin_amdgcn_raw_buffer_load_b32(rsx, vsc, ((mt0 + j) * nsteps + s) * 64, 0);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step = 8 rows (group g = 0, 1; weight tile i = 0..3), each row 4
  // integer MFMAs (P) and 4 scale MFMAs (S) and then 16 convert + FMA pairs
  // on the VALU.  The rows are software-pipelined: row r + 1's MFMAs are
  // issued one by one between row r's dequant FMAs (P and S double-
  // buffered), fenced so the compiler keeps that order, so the matrix core
  // runs while the VALU dequantizes instead of each waiting on the other.
  auto compute = [&](const Ops& o) {
    // scale-MFMA operands: A row n holds (s_w[n][g0], s_w[n][g1]) at k = 0, 1;
    // B column m holds s_x[m][g] at k = g, so A B = s_w[n][g] s_x[m][g]
    f16x4 sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = __builtin_bit_cast(f16x4, u32x2{o.sw[i] & mk0, 0u});
    i32x4 ub[4];
    f16x4 sb[4];
    auto token_side = [&](int g) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ub[j] = widen_nibbles(o.b[j][2 * g], o.b[j][2 * g + 1]);
        sb[j] = __builtin_bit_cast(f16x4, u32x2{o.sx[j] & (g ? mg1 : mg0), 0u});
      }
    };
    i32x4 P[2][4];
    f32x4 S[2][4];
    i32x4 ua;
    auto mfma_pair = [&](int buf, int i, int j) {
      P[buf][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ua, ub[j], i32x4{0, 0, 0, 0}, 0, 0, 0);
      S[buf][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(sa[i], sb[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    };
    token_side(0);
    ua = widen_nibbles(o.a[0][0], o.a[0][1]);
#pragma unroll
    for (int j = 0; j < 4; ++j) mfma_pair(0, 0, j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int c = r & 1, i = r & 3;
      const int r1 = r + 1, g1 = r1 >> 2, i1 = r1 & 3;
      if (r1 < 8) {
        if (i1 == 0) token_side(g1);
        ua = widen_nibbles(o.a[i1][2 * g1], o.a[i1][2 * g1 + 1]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (r1 < 8) mfma_pair(c ^ 1, i1, j);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) acc[i][j][q4] = __builtin_fmaf(float(P[c][j][q4]), S[c][j][q4], acc[i][j][q4]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // two-step software pipeline: step s + 1's loads are in flight while step
  // s computes (the last step reloads itself, so every trip is the same)
  Ops o0, o1;
  load(o0, 0);
  int s = 0;
  for (; s + 2 <= nsteps; s += 2) {
    load(o1, s + 1);
    compute(o0);
    load(o0, s + 2 < nsteps ? s + 2 : nsteps - 1);
    compute(o1);
  }
  if (s < nsteps) compute(o0);

  // epilogue: + T L2 (16-bit MFMA into a separate accumulator, added on the
  // VALU so the dequant accumulators stay in VGPRs), + bias, GELU, round, store
  f32x4 lr[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) lr[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4* l2 = reinterpret_cast<const u32x4*>(p.l2);
  const u32x4* tt = reinterpret_cast<const u32x4*>(p.t);
  for (int c = 0; c < p.nchunks; ++c) {
    u32x4 la[4], tb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) la[i] = l2[((nt0 + i) * (p.slots / 32) + c) * 64 + lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) tb[j] = tt[((mt0 + j) * (p.slots / 32) + c) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) lr[i][j] = mfma16<DT>(la[i], tb[j], lr[i][j]);
  }
  // the wave's 64 x 64 tile goes through LDS as [token][column] rows so the
  // global stores cover whole 128-byte lines (non-temporal: Y is not read
  // again here)
  constexpr int OP = 64 * 2 + 16;                       // bytes per staged row
  __shared__ __attribute__((aligned(16))) uint8_t ostage[4][64 * OP];
  uint8_t* ob = ostage[wave];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 bv = *reinterpret_cast<const f32x4*>(p.bias + n0 + 16 * i + 4 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // acc holds 256 x the dequantized sum; acc 2^-8 + lr is one rounding
        v[r] = __builtin_fmaf(acc[i][j][r], 1.0f / 256.0f, lr[i][j][r]) + bv[r];
        if constexpr (GELU) v[r] = gelu_erf(v[r]);
      }
      *reinterpret_cast<u32x2*>(ob + (16 * j + (lane & 15)) * OP + (16 * i + 4 * q) * 2) =
          u32x2{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
    }
  }
  SVDQ_WAIT_LGKM0();
  if (!CHAIN || p.Y != nullptr) {
    // 8 rows of 128 bytes per instruction: lane l takes row l / 8, piece l % 8
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = 8 * it + (lane >> 3), col = (lane & 7) * 8;
      const u32x4 val = *reinterpret_cast<const u32x4*>(ob + row * OP + col * 2);
      if (m0 + row < p.M) __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(p.Y + (m0 + row) * p.ldy + n0 + col));
    }
  }
  if constexpr (CHAIN) {
    __syncthreads();                      // every wave's tile is staged
    int4_chain_epilogue<DT>(p, &ostage[0][0], wave, lane);
  }
  trace_mark(p.trace, 2);
}


// ------------------------------------------------------------------- k1_w8
// INT8 activation kernel (the 8-bit setting: one scale per token over all
// of K, so a token's maximum must be known before any of its codes).  One
// workgroup = 16 tokens; its four waves take the 128-deep steps round robin
// in the INT4 lane layout (lane m + 16q holds k in [32c + 8q, +8) of chunk
// c), so L1x uses the INT4 tiling.  Pass 1 streams X: the running max
// of |x_hat| and the down-projection T on the 16 x 16 x 32 MFMA.  The token
// maxima meet across the four lanes of a token and the four waves in LDS.
// Pass 2 streams the workgroup's X again (96 KB at K = 3072, mostly from L2)
// and writes the codes; each lane's 8 codes of a chunk are 8 contiguous
// bytes of the INT8 fragment the GEMM (k2_mx with I8) reads.  Both passes keep the next step's loads in
// flight; rows past M repeat row M - 1.  X is loaded row-contiguously and
// passed through the wave's LDS buffer into the lane map, and the outputs
// leave with non-temporal stores, as in k1_act.
template <int DT, int NJT>
__global__ __launch_bounds__(256, 2) void k1_w8(K1Params p) {
  __shared__ float smax[4][16];
  __shared__ f32x4 red[4][NJT > 0 ? NJT : 1][64];
  __shared__ __attribute__((aligned(16))) uint8_t xbuf[4][4096];   // the waves' step buffers
  const int mt = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  const int64_t row = min(int64_t(mt) * 16 + m, p.M - 1);
  const int nsteps = int(p.K / KSTEP);
  const int nmine = (nsteps - wave + 3) / 4;
  (void)row;
  // load c's row (4c + lane / 16) and the piece this lane loads, (lane % 16)
  // ^ row, as element offsets from the tile's first row
  const uint16_t* xtile = p.X + int64_t(mt) * 16 * p.ldx;
  int xo[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = 4 * c + (lane >> 4);
    xo[c] = int(min(int64_t(mt) * 16 + r, p.M - 1) - int64_t(mt) * 16) * int(p.ldx) + 8 * ((lane & 15) ^ r);
  }
  const int njc = p.njt > 0 ? p.njt - 1 : 0;
  auto step_of = [&](int i) { return nmine > 0 ? wave + 4 * (i < nmine ? i : nmine - 1) : 0; };
  auto load_x = [&](u32x4 (&x)[4], int i) {
    const int s = step_of(i);
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = *reinterpret_cast<const u32x4*>(xtile + (xo[c] + s * KSTEP));
  };
  // a landed step through the wave's LDS buffer into the lane map (piece
  // 4c + q of row m sits at position (4c + q) ^ m)
  uint8_t* xb = xbuf[wave];
  auto to_lane_map = [&](u32x4 (&x)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<u32x4*>(xb + (4 * c + (lane >> 4)) * 256 + 16 * (lane & 15)) = x[c];
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = *reinterpret_cast<const u32x4*>(xb + m * 256 + 16 * ((4 * c + q) ^ m));
  };
  auto load_l1x = [&](u32x4 (&l)[NJT > 0 ? NJT : 1][4], int i) {
    const int s = step_of(i);
    const u32x4* l1 = reinterpret_cast<const u32x4*>(p.l1x) + (size_t(s) * (p.slots / 16)) * 4 * 64 + lane;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
      for (int c = 0; c < 4; ++c) l[jt][c] = l1[((jt < njc ? jt : njc) * 4 + c) * 64];
  };
  // x_hat = x * invlambda (one fp32 multiply) for chunk c of step s, the
  // same values in both passes
  auto smooth_c = [&](const u32x4& xc, int s, int c, float (&xh)[8]) {
    const int k = s * KSTEP + 32 * c + 8 * q;
    const f32x4 il0 = *reinterpret_cast<const f32x4*>(p.invlam + k);
    const f32x4 il1 = *reinterpret_cast<const f32x4*>(p.invlam + k + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x4& il = e < 2 ? il0 : il1;
      xh[2 * e] = h2f<DT>(xc[e] & 0xFFFFu) * il[(2 * e) & 3];
      xh[2 * e + 1] = h2f<DT>(xc[e] >> 16) * il[(2 * e + 1) & 3];
    }
  };
  f32x4 tacc[NJT > 0 ? NJT : 1];
#pragma unroll
  for (int j = 0; j < NJT; ++j) tacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float am = 0.0f;
  auto pass1_step = [&](const u32x4 (&x)[4], const u32x4 (&l)[NJT > 0 ? NJT : 1][4], int i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float xh[8];
      smooth_c(x[c], step_of(i), c, xh);
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(xh[e]));
    }
    if (i < nmine) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int c = 0; c < 4; ++c) tacc[jt] = mfma16<DT>(l[jt][c], x[c], tacc[jt]);
    }
  };
  if constexpr (NJT <= 4) {
    u32x4 xa[4], xb2[4];
    u32x4 la[NJT > 0 ? NJT : 1][4], lb[NJT > 0 ? NJT : 1][4];
    load_l1x(la, 0);
    load_x(xa, 0);
    for (int i = 0; i < nmine; i += 2) {
      load_l1x(lb, i + 1);
      load_x(xb2, i + 1);
      to_lane_map(xa);
      pass1_step(xa, la, i);
      load_l1x(la, i + 2);
      load_x(xa, i + 2);
      to_lane_map(xb2);
      pass1_step(xb2, lb, i + 1);
    }
  } else {
    // ranks above 64: the wide L1x is loaded once per step, after X
    u32x4 xa[4];
    u32x4 la[NJT][4];
    for (int i = 0; i < nmine; ++i) {
      load_x(xa, i);
      load_l1x(la, i);
      to_lane_map(xa);
      pass1_step(xa, la, i);
    }
  }
  am = quad_max(am);
  if (q == 0) smax[wave][m] = am;
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt) red[wave][jt][lane] = tacc[jt];
  __syncthreads();
  const float tmax = fmaxf(fmaxf(smax[0][m], smax[1][m]), fmaxf(smax[2][m], smax[3][m]));
  const float sc = tmax / 127.0f;
  const float inv = sc != 0.0f ? 1.0f / sc : 0.0f;
  // below 2^-128 the reciprocal overflows: such a token takes the division
  // for every code
  const bool inv_inf = !(inv <= 3.40282347e38f);
  if (wave == 0 && q == 0) __builtin_nontemporal_store(sc, reinterpret_cast<float*>(p.sx) + size_t(mt) * 16 + m);
  if constexpr (NJT > 0) {
    // T = the four waves' partial sums (fixed order), rounded once, in the
    // GEMM's low-rank layout (32-row tiles, 16-rank chunks); lane holds
    // T[m][16 jt + 4q + i]
    for (int jt = wave; jt < p.njt; jt += 4) {
      f32x4 v = red[0][jt][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) v += red[w][jt][lane];
      const int t32 = mt >> 1, r32 = 16 * (mt & 1) + m;
      uint16_t* dst = p.t + ((size_t(t32) * (p.slots / 16) + jt) * 64 + r32 + 32 * (q >> 1)) * 8 + 4 * (q & 1);
      __builtin_nontemporal_store(u32x2{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])}, reinterpret_cast<u32x2*>(dst));
    }
  }
  // pass 2: codes rint(x_hat / s), from x_hat * (1/s) except for lanes whose
  // quotient lies within 2^-15 of a half-integer (|x_hat / s| <= 127 keeps
  // x_hat * fl(1/s) within 2^-16 of fl(x_hat / s)), which redo it with the
  // correctly rounded division; clamp to +-127
  auto pass2_step = [&](const u32x4 (&x)[4], int i) {
    const int s = step_of(i);
    const int nst64 = int(p.K / 64);
    const int t32 = mt >> 1, r32 = 16 * (mt & 1) + m;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float xh[8], r[8];
      smooth_c(x[c], s, c, xh);
      bool near = inv_inf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = xh[e] * inv;
        r[e] = rintf(qv);
        near |= fabsf(qv - r[e]) >= 0.5f - 0x1p-15f;
      }
      if (__builtin_expect(near, 0)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = sc != 0.0f ? rintf(xh[e] / sc) : 0.0f;
      }
      unsigned d[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float rc = __builtin_amdgcn_fmed3f(r[e], -127.0f, 127.0f);   // clamp, one v_med3_f32
        d[e >> 2] |= (unsigned(int(rc)) & 0xFFu) << (8 * (e & 3));
      }
      // k = 128 s + 32 c + 8 q + e: 64-deep step 2s + c/2, half c % 2, lane
      // (row in the 32-row tile) + 32 (q / 2), byte 8 (q % 2) + e
      const size_t frag = ((size_t(t32) * nst64 + 2 * s + (c >> 1)) * 2 + (c & 1)) * 64 + r32 + 32 * (q >> 1);
      __builtin_nontemporal_store(u32x2{d[0], d[1]}, reinterpret_cast<u32x2*>(p.xq + frag * 16 + 8 * (q & 1)));
    }
  };
  {
    u32x4 xa[4], xb2[4];
    load_x(xa, 0);
    for (int i = 0; i < nmine; i += 2) {
      load_x(xb2, i + 1);
      to_lane_map(xa);
      pass2_step(xa, i);
      load_x(xa, i + 2);
      to_lane_map(xb2);
      pass2_step(xb2, i + 1);
    }
  }
}

// ------------------------------------------------------------ k2_mx (MXFP4)
// One workgroup = 256 output columns x 256 tokens, 4 waves in a 2 x 2 grid,
// each 128 x 128 = 4 x 4 tiles of 32 x 32 on V_MFMA_SCALE_F32_32X32X64_F8F6F4
// (16 fp32 accumulators per tile and lane, 256 in all).  Per 128-deep K
// step the workgroup stages 8 weight and 8 activation fragment tiles (2 KB
// each) and their e8m0 scale dwords (34 KB) in LDS with direct global->LDS
// loads; mx::STAGES steps are in flight and the fragments of the next step
// are read into registers while the current step's 32 MFMAs run.  The tile
// order is XCD-aware: consecutive tiles of a grouped order share an XCD's L2.
// The accumulators start at the bias (one 16-bit MFMA per 32 x 32 tile); the
// up-projection T L2 runs as extra pipeline steps on the 32 x 32 x 16
// bf16/f16 MFMA; the epilogue applies GELU if asked, rounds, and writes the
// tile through LDS so every global store covers whole rows.
namespace mx {
constexpr int STAGES = 4;
constexpr int A_OFF = 0;                 // 8 weight tiles x 2 halves x 1 KB
constexpr int B_OFF = 16 * 1024;         // 8 activation tiles x 2 halves x 1 KB
constexpr int SA_OFF = 32 * 1024;        // 4 weight scale dwords x 64 lanes
constexpr int SB_OFF = 32 * 1024 + 1024; // 4 activation scale dwords x 64 lanes
constexpr int STAGE_BYTES = 34 * 1024;
constexpr int GROUP_M = 8;               // m-tiles per group of the tile order
constexpr int OUT_PITCH = 272;           // bytes per staged output row (128 x 2 + 16)
}  // namespace mx
static_assert(4 * 128 * mx::OUT_PITCH <= mx::STAGES * mx::STAGE_BYTES, "output staging must fit the LDS ring");

// Slot plan of a steady K step (32 MFMAs): global->LDS load d after MFMA
// 3d + 1, LDS read e in the remaining slots in order.
__host__ __device__ constexpr int dma_slot(int k) { return (k % 3 == 1 && k <= 28) ? k / 3 : -1; }
__host__ __device__ constexpr int lds_slot(int k) {
  int c = 0;
  for (int i = 0; i < k; ++i) c += dma_slot(i) < 0 ? 1 : 0;
  return dma_slot(k) < 0 ? c : -1;
}
static_assert(dma_slot(28) == 9 && lds_slot(26) == 17, "every load and read has a slot");

struct MxParams {
  const uint8_t* wq;
  const uint8_t* sw;
  const uint16_t* l2;
  const float* bias;
  const uint8_t* xq;
  const uint8_t* sx;
  const uint16_t* t;
  uint16_t* Y;
  int64_t ldy, M, N, K;
  int slots, nchunks16;
  int tiles_n, tiles_m;
  int tiles_m_pad32;     // 32-row token tiles in the workspace (its padded rows / 32)
  // byte offsets of the weight-side regions from l2 (all in the layer blob)
  // and of the token-side regions from xq (all in the workspace); both spans
  // are below 2 GiB, so the stage loads take them as scalar offsets
  int off_wq, off_sw, off_sx, off_t;
  unsigned long long* trace;   // GEMM trace records (SVDQ_FLAG_TRACE) or null
  // Epilogue chaining (CHAIN): this layer's output is the next layer's
  // input.  nx_invlam: the next layer's 1/lambda over this layer's N
  // columns; nx_l1x: its L1x in the activation kernel's tiling; nx_xq,
  // nx_sx: its workspace codes and scales (written here); nx_tp: fp32
  // partial down-projections [tiles_n][nx_Mp][nx_slots], one slab per
  // column tile of this layer (256 columns in k2_mx, 192 in k2_mx8; summed
  // by k_tfin).
  const float* nx_invlam;
  const uint16_t* nx_l1x;
  uint8_t* nx_xq;
  uint8_t* nx_sx;
  float* nx_tp;
  int64_t nx_Mp;
  int nx_slots, nx_njt;
  // staggered start: the odd-indexed ones among the first stagger_wgs
  // workgroups sleep stagger_sleeps x 8128 clocks before their first tile
  int stagger_wgs, stagger_sleeps;
  // k2_mx: XCD x (the workgroups with index % 8 == x) takes tiles
  // [xcd_start[x], xcd_start[x] + xcd_count[x]) of the grouped order; its
  // workgroups past the count have no tile
  int xcd_start[8], xcd_count[8];
};

// Staggered start.  Workgroups are dealt to the XCDs round robin, so the
// odd-indexed workgroups of the first round are those of the odd XCDs.
// Holding them back for a few microseconds keeps the two halves of the chip
// out of phase for the rest of the launch: one half's epilogues and stores
// fall inside the other half's K loops instead of every tile switching
// between the matrix-core phase and the store phase at once, and the
// power-limited clock runs higher.  FLUX fc1, MXFP4, one box, one process:
// 0 / 1 / 2 / 3 / 4 sleeps of 8128 clocks give 101.7 / 96.7 / 94.6 / 95.9 /
// 99.5 us, the tiles' clock 1.81 -> 2.06 GHz at 2; the delay itself is paid
// once, so launches of fewer than three rounds gain nothing (FLUX QKV, 2.5
// rounds: +1%).  Staggering half of every XCD instead is slower than none.
__device__ __forceinline__ void stagger_start(int wgs, int sleeps) {
  if (int(blockIdx.x) < wgs && (blockIdx.x & 1))
    for (int i = 0; i < sleeps; ++i) __builtin_amdgcn_s_sleep(127);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

template <bool B> struct BoolTag { static constexpr bool value = B; };

// Scaled FP4 32x32x64 MFMA with the scale bytes picked by op_sel; oa / ob are
// compile-time constants at every call site (unrolled loops), so the switch folds.
__device__ __forceinline__ f32x16 mfma_mx32(const i32x8& a, const i32x8& b, f32x16 c, int sa, int sb, int oa, int ob) {
#define SVDQ_MX_CASE(OA, OB) \
  case OA * 4 + OB: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, OA, sa, OB, sb);
  switch (oa * 4 + ob) {
    SVDQ_MX_CASE(0, 0) SVDQ_MX_CASE(0, 1) SVDQ_MX_CASE(0, 2) SVDQ_MX_CASE(0, 3)
    SVDQ_MX_CASE(1, 0) SVDQ_MX_CASE(1, 1) SVDQ_MX_CASE(1, 2) SVDQ_MX_CASE(1, 3)
    SVDQ_MX_CASE(2, 0) SVDQ_MX_CASE(2, 1) SVDQ_MX_CASE(2, 2) SVDQ_MX_CASE(2, 3)
    SVDQ_MX_CASE(3, 0) SVDQ_MX_CASE(3, 1) SVDQ_MX_CASE(3, 2) SVDQ_MX_CASE(3, 3)
    default: return c;
  }
#undef SVDQ_MX_CASE
}

template <int DT>
__device__ __forceinline__ f32x16 mfma32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == SVDQ_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}



// Epilogue chaining: the staged 16-bit output tile (the exact bits the
// layer would store) is the next layer's input, so its activation kernel
// pass is done here.  Per wave (128 tokens x 128 columns = one 128-deep K
// step of the next layer):
//  * codes and scales: lane l takes token 32t + l % 32 and block
//    b = 2h + l / 32 of the step -- exactly one 16-byte piece of the next
//    layer's fragment and one byte of its scale dword -- and applies the
//    activation kernel's rule (x_hat = x * invlambda in fp32, e8m0 of the
//    block absmax, E2M1 codes);
//  * down-projection: after a workgroup barrier, wave (wm, wn) sums
//    x L1x over all 256 columns of the tile (its own and its neighbour's
//    staged halves) for tokens 64 wn .. 64 wn + 63 of the pair's 128, on
//    the 16 x 16 x 32 MFMA with L1x as the A operand, and writes the fp32
//    result to this column tile's slab.
template <int DT>
__device__ __forceinline__ void chain_epilogue(const MxParams& p, const uint8_t* smem, const uint8_t* ob, int wave,
                                               int lane, int64_t m0, int64_t n0, int64_t nw, int64_t mw) {
  const int wn = wave & 1, wm = wave >> 1;
  const int nst = int(p.N / KSTEP);        // K steps of the next layer
  if (nw < p.N) {
    const int s2 = int(nw / KSTEP), half = lane >> 5, r32 = lane & 31;
    unsigned sdw[2] = {0u, 0u};            // scale dwords of the two 32-tile pairs
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int b = 2 * h + half;
      f32x4 il[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) il[e] = *reinterpret_cast<const f32x4*>(p.nx_invlam + nw + 32 * b + 4 * e);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint8_t* src = ob + (32 * t + r32) * mx::OUT_PITCH + 64 * b;
        float xh[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(src + 16 * i);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int x = 8 * i + 2 * e;
            xh[x] = h2f<DT>(v[e] & 0xFFFFu) * il[x >> 2][x & 3];
            xh[x + 1] = h2f<DT>(v[e] >> 16) * il[(x + 1) >> 2][(x + 1) & 3];
          }
        }
        float am = 0.0f;
#pragma unroll
        for (int x = 0; x < 32; ++x) am = fmaxf(am, fabsf(xh[x]));
        const int ex = e8m0_needs_slow(am) ? e8m0_slow(am) : e8m0_fast(am);
        const float scl = ex != 0 ? __uint_as_float(unsigned(ex) << 23) : 1.0f;
        unsigned d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unsigned v = 0u;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const unsigned cv = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, xh[8 * i + 2 * bb], xh[8 * i + 2 * bb + 1], scl, 0);
            v |= (cv & 0xFFu) << (8 * bb);
          }
          d[i] = v;
        }
        const int64_t tg = mw / 32 + t;
        *reinterpret_cast<u32x4*>(p.nx_xq + ((size_t(tg) * nst + s2) * 2 + h) * 1024 + lane * 16) = u32x4{d[0], d[1], d[2], d[3]};
        sdw[t >> 1] |= unsigned(ex) << (8 * (2 * (t & 1) + h));
      }
    }
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
      reinterpret_cast<unsigned*>(p.nx_sx)[(size_t(mw / 64 + tp) * nst + s2) * 64 + lane] = sdw[tp];
  }
  if (p.nx_njt == 0) return;               // uniform over the workgroup
  __syncthreads();                         // both halves of the pair are staged
  const int cs = p.nx_slots / 16;
  const int nblk = n0 + 128 < p.N ? 2 : 1; // column halves of the tile inside N
  const u32x4* l1x = reinterpret_cast<const u32x4*>(p.nx_l1x);
  float* tp = p.nx_tp + (size_t(n0 / 256) * p.nx_Mp + mw + 64 * wn) * p.nx_slots;
  const int q = lane >> 4;
  for (int jt = 0; jt < p.nx_njt; ++jt) {
    u32x4 la[2][4];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        la[x][c] = x < nblk ? l1x[((size_t(n0 / KSTEP + x) * cs + jt) * 4 + c) * 64 + lane] : u32x4{0u, 0u, 0u, 0u};
    // the four 16-token blocks accumulate side by side (four independent
    // MFMA chains instead of one)
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (x < nblk) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            // MFMA c takes k in [32q + 8c, +8) from lane group q (the MXFP4 L1x tiling)
            const int row = 64 * wn + 16 * u + (lane & 15);
            const uint8_t* src = smem + (2 * wm + x) * (128 * mx::OUT_PITCH) + row * mx::OUT_PITCH + 64 * q + 16 * c;
            acc[u] = mfma16<DT>(la[x][c], *reinterpret_cast<const u32x4*>(src), acc[u]);
          }
      }
    }
    // lane holds T[token row][16 jt + 4 q + i]
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<f32x4*>(tp + size_t(16 * u + (lane & 15)) * p.nx_slots + 16 * jt + 4 * q) = acc[u];
  }
}

template <int DT, bool GELU, bool CHAIN = false, bool I8 = false>
__global__ __launch_bounds__(256) void k2_mx(MxParams p) {
  trace_mark(p.trace, 0);
  stagger_start(p.stagger_wgs, p.stagger_sleeps);
  // one LDS object (a second one makes the compiler wait for every global->LDS
  // load before any LDS read)
  // (the ring, then each wave's 128 bias values)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[mx::STAGES * mx::STAGE_BYTES + 4 * 512];
  // the wave index is uniform: keep it (and every LDS address derived from it) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wn = wave & 1, wm = wave >> 1;
  // I8: the 8-bit setting on the same pipeline -- a step is 64 deep (2 KB
  // of int8 codes per 32-row tile, like an MXFP4 128-deep step), the
  // 32 x 32 x 32 int8 MFMA chains int32 accumulators, no scale loads
  constexpr int LPS = I8 ? 8 : 10;         // global->LDS loads per wave and step
  const int nsteps = int(p.K / (I8 ? 64 : KSTEP));
  const int64_t ntiles_n = p.N / 32;       // valid 32-row weight tiles
  const int cs = p.slots / 16;              // 16-rank chunks per tile in L2 / T

  // fragments of one step in registers (double-buffered across steps)
  struct Frags {
    u32x4 a[4][2], b[4][2];
    int sa0, sa1, sb0, sb1;
  };
  f32x16 acc[4][4];

  {
    // XCD-aware tile index: workgroups are dealt to the 8 XCDs round robin,
    // so give XCD x a contiguous range of the tile order (they share its L2)
    const int bid = blockIdx.x;
    const int xcd = bid & 7, kx = bid >> 3;
    if (kx >= p.xcd_count[xcd]) {          // no tile (uniform over the workgroup)
      trace_mark(p.trace, 2);
      return;
    }
    const int tile = p.xcd_start[xcd] + kx;
    // grouped tile order: GROUP_M m-tiles sweep the n-tiles
    const int gsz_full = mx::GROUP_M * p.tiles_n;
    const int grp = tile / gsz_full, first_m = grp * mx::GROUP_M;
    const int gm = (p.tiles_m - first_m) < mx::GROUP_M ? (p.tiles_m - first_m) : mx::GROUP_M;
    const int within = tile - grp * gsz_full;
    const int tm = first_m + within % gm, tn = within / gm;
    const int64_t n0 = int64_t(tn) * 256, m0 = int64_t(tm) * 256;
    // After the K steps come "low-rank steps": each stages two 16-rank chunks
    // of L2 (weight side) and T (token side) through the same pipeline, and
    // runs the up-projection on the 16-bit MFMA into the same accumulators.
    const int nk = nsteps;
    const int total = nk + (p.nchunks16 + 1) / 2;

    int64_t tA[4], tB[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int u = 4 * wave + f;
      const int64_t nt = n0 / 32 + u / 2;
      tA[f] = nt < ntiles_n ? nt : ntiles_n - 1;   // a partial last tile re-reads a valid tile
      tB[f] = m0 / 32 + u / 2;
    }
    int64_t pn = n0 / 64 + wave;
    pn = pn < p.N / 64 ? pn : p.N / 64 - 1;
    const int osa = p.off_sw + int(pn * nsteps) * 256;
    const int osb = p.off_sx + int((m0 / 64 + wave) * nsteps) * 256;
    // Stage loads are buffer loads straight into LDS: one descriptor over the
    // blob (L2, codes, scales), one over the workspace (codes, scales, T);
    // each load takes a scalar byte offset plus the lane's offset, so no
    // 64-bit per-lane address is computed or kept in vector registers.
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)p.l2, 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc((void*)p.xq, 0, -1, 0x00020000);
    const int lo16 = lane * 16, lo4 = lane * 4;
    auto dma16 = [&](__amdgpu_buffer_rsrc_t rs, int soff, uint8_t* dst) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, lo16, soff, 0, 0);
    };
    auto dma4 = [&](__amdgpu_buffer_rsrc_t rs, int soff, uint8_t* dst) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 4, lo4, soff, 0, 0);
    };
    // this wave's fixed source offsets; step r adds r * 2048 (fragments)
    // or r * 256 (scales)
    int ga[4], gb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int h = (4 * wave + f) & 1;
      ga[f] = p.off_wq + int(tA[f] * nsteps * 2 + h) * 1024;
      gb[f] = int(tB[f] * nsteps * 2 + h) * 1024;
    }
    // one of the 10 loads a wave issues per K step
    auto issue_unit = [&](int r, uint8_t* base, int x) {
      if (I8 && x >= 8) return;
      if (x < 4) dma16(rsb, ga[x] + r * 2048, base + mx::A_OFF + (4 * wave + x) * 1024);
      else if (x < 8) dma16(rsw, gb[x - 4] + r * 2048, base + mx::B_OFF + (4 * wave + x - 4) * 1024);
      else if (x == 8) dma4(rsb, osa + r * 256, base + mx::SA_OFF + wave * 256);
      else dma4(rsw, osb + r * 256, base + mx::SB_OFF + wave * 256);
    };
    // the 10 loads of low-rank step e: chunks 2e, 2e+1 of L2 and T (the scale
    // slots reload the first step's scales so every step issues 10 loads)
    auto issue_lr = [&](int e, uint8_t* base) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int h = (4 * wave + f) & 1;
        int c = 2 * e + h;
        c = c < p.nchunks16 ? c : p.nchunks16 - 1;
        dma16(rsb, int(tA[f] * cs + c) * 1024, base + mx::A_OFF + (4 * wave + f) * 1024);
        dma16(rsw, p.off_t + int(tB[f] * cs + c) * 1024, base + mx::B_OFF + (4 * wave + f) * 1024);
      }
      if constexpr (!I8) {
        dma4(rsb, osa, base + mx::SA_OFF + wave * 256);
        dma4(rsw, osb, base + mx::SB_OFF + wave * 256);
      }
    };
    auto issue = [&](int r, int st) {
      uint8_t* base = smem + st * mx::STAGE_BYTES;
      if (r < nk) {
#pragma unroll
        for (int x = 0; x < LPS; ++x) issue_unit(r, base, x);
      } else {
        issue_lr(r - nk, base);
      }
    };
    auto read_frags = [&](Frags& F, int st, bool scales = true) {   // (a low-rank step has no scales)
      const uint8_t* base = smem + st * mx::STAGE_BYTES;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          F.b[j][h] = *reinterpret_cast<const u32x4*>(base + mx::B_OFF + ((4 * wm + j) * 2 + h) * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          F.a[i][h] = *reinterpret_cast<const u32x4*>(base + mx::A_OFF + ((4 * wn + i) * 2 + h) * 1024 + lane * 16);
      if (!I8 && scales) {
        F.sb0 = *reinterpret_cast<const int*>(base + mx::SB_OFF + (2 * wm) * 256 + lane * 4);
        F.sb1 = *reinterpret_cast<const int*>(base + mx::SB_OFF + (2 * wm + 1) * 256 + lane * 4);
        F.sa0 = *reinterpret_cast<const int*>(base + mx::SA_OFF + (2 * wn) * 256 + lane * 4);
        F.sa1 = *reinterpret_cast<const int*>(base + mx::SA_OFF + (2 * wn + 1) * 256 + lane * 4);
      }
    };
    // One MFMA of a K step (k = 0..31 walks h, i, j; the two halves of a
    // tile's K are 16 MFMAs apart, so no MFMA waits on its predecessor).
    auto mfma_k = [&](const Frags& F, int k) {
      const int h = k >> 4, i = (k >> 2) & 3, j = k & 3;
      if constexpr (I8) {
        acc[i][j] = __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
            __builtin_bit_cast(i32x4, F.a[i][h]), __builtin_bit_cast(i32x4, F.b[j][h]),
            __builtin_bit_cast(i32x16, acc[i][j]), 0, 0, 0));
        return;
      }
      const i32x8 a = i32x8{int(F.a[i][h][0]), int(F.a[i][h][1]), int(F.a[i][h][2]), int(F.a[i][h][3]), 0, 0, 0, 0};
      const i32x8 b = i32x8{int(F.b[j][h][0]), int(F.b[j][h][1]), int(F.b[j][h][2]), int(F.b[j][h][3]), 0, 0, 0, 0};
      acc[i][j] = mfma_mx32(a, b, acc[i][j], i < 2 ? F.sa0 : F.sa1, j < 2 ? F.sb0 : F.sb1, 2 * (i & 1) + h, 2 * (j & 1) + h);
    };
    auto compute = [&](const Frags& F) {
#pragma unroll
      for (int k = 0; k < 32; ++k) mfma_k(F, k);
    };
    // up-projection of low-rank step e: chunks 2e, 2e+1 of T L2
    auto compute_lr = [&](int e, const Frags& F) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (2 * e + h < p.nchunks16) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x16<DT>(F.a[i][h], F.b[j][h], acc[i][j]);
        }
    };
    // Memory op k of the next step, placed after MFMA k.  The 10 global->LDS
    // loads of step r + 3 go after every third MFMA (k = 1, 4, ..., 28) so the
    // four waves never queue more than the texture path drains per MFMA; the
    // other slots take the 8 token and 8 weight fragment reads of step r + 1,
    // then its 4 scale reads.
    auto mem_k = [&](Frags& nxt, const uint8_t* rb, uint8_t* lb, int r3, int k) {
      const int d = dma_slot(k);
      if (d >= 0) {
        issue_unit(r3, lb, d);
        return;
      }
      const int e = lds_slot(k);
      if (e < 8) {
        nxt.b[e >> 1][e & 1] = *reinterpret_cast<const u32x4*>(rb + mx::B_OFF + ((4 * wm + (e >> 1)) * 2 + (e & 1)) * 1024 + lane * 16);
      } else if (e < 16) {
        const int ee = e - 8;
        nxt.a[ee >> 1][ee & 1] = *reinterpret_cast<const u32x4*>(rb + mx::A_OFF + ((4 * wn + (ee >> 1)) * 2 + (ee & 1)) * 1024 + lane * 16);
      } else if (I8) {
        return;
      } else if (e == 16) {
        nxt.sb0 = *reinterpret_cast<const int*>(rb + mx::SB_OFF + (2 * wm) * 256 + lane * 4);
        nxt.sb1 = *reinterpret_cast<const int*>(rb + mx::SB_OFF + (2 * wm + 1) * 256 + lane * 4);
      } else if (e == 17) {
        nxt.sa0 = *reinterpret_cast<const int*>(rb + mx::SA_OFF + (2 * wn) * 256 + lane * 4);
        nxt.sa1 = *reinterpret_cast<const int*>(rb + mx::SA_OFF + (2 * wn + 1) * 256 + lane * 4);
      }
    };
    // Iteration r: wait until step r+1 is in LDS (its own loads, then the
    // barrier for everyone's), then run step r's 32 MFMAs with the reads of
    // step r+1 and the refill of step r's own stage (with step r+4) placed
    // between them, fenced so the compiler keeps that order.  Step r's
    // fragments were read into registers during iteration r-1 and every
    // wave retired those reads before this barrier, so its stage is free:
    // all four stages hold steps in flight, and a step's loads get three
    // iterations to land.
    auto body_full = [&](int r, Frags& cur, Frags& nxt) {   // needs r + 4 < nk
      // cur's LDS reads were issued an iteration ago; retire them here so the
      // 20 reads below need no counter slot (lgkmcnt counts at most 15)
      SVDQ_WAIT_LGKM0();
      SVDQ_WAIT_VM(2 * LPS);                 // steps r+2 and r+3 may stay in flight
      __builtin_amdgcn_s_barrier();
      const uint8_t* rb = smem + ((r + 1) & 3) * mx::STAGE_BYTES;
      uint8_t* lb = smem + (r & 3) * mx::STAGE_BYTES;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        mfma_k(cur, k);
        mem_k(nxt, rb, lb, r + 4, k);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // the last K steps: wait for step r+1 (if it is a K step), refill step
    // r's stage with step r+4, read step r+1, compute step r
    auto body_tail = [&](int r, Frags& cur, Frags& nxt) {
      SVDQ_WAIT_LGKM0();
      if (r + 1 < nk) {
        const int after = (r + 2 < total ? 1 : 0) + (r + 3 < total ? 1 : 0);   // steps requested after r+1
        if (after == 2) SVDQ_WAIT_VM(2 * LPS);
        else if (after == 1) SVDQ_WAIT_VM(LPS);
        else SVDQ_WAIT_VM(0);
        __builtin_amdgcn_s_barrier();
        if (r + 4 < total) issue(r + 4, r & 3);
        read_frags(nxt, (r + 1) & 3);
      } else if (r + 4 < total) {
        // the last K step still requests step r + 4 (a low-rank step):
        // after this barrier every wave has retired its reads of step r
        __builtin_amdgcn_s_barrier();
        issue(r + 4, r & 3);
      }
      compute(cur);
    };
    static_assert(mx::STAGES == 4, "the step bookkeeping assumes a 4-stage ring");

    // The bias of this wave's 128 columns goes to LDS by the same buffer
    // loads as the stages, issued before them so the prologue's wait for
    // the first stage covers it.  (Loaded into registers, the compiler's
    // wait before the first use would also wait for every stage issued
    // after it.)  Lane l < 32 then takes column 32i + l.
    float* bias_lds = reinterpret_cast<float*>(smem + mx::STAGES * mx::STAGE_BYTES + wave * 512);
    {
      const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc((void*)p.bias, 0, -1, 0x00020000);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t nb = n0 + 128 * wn + 64 * h + lane;
        nb = nb < p.N ? nb : p.N - 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbias, (lds_ptr_t)(bias_lds + 64 * h), 4, int(nb) * 4, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < mx::STAGES; ++r)
      if (r < total) issue(r, r);
    float bcol[4];
    auto read_bias = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i) bcol[i] = bias_lds[32 * i + (lane & 31)];
    };
    // Accumulators start at the bias: one 32 x 32 x 16 MFMA per tile with a
    // zero C operand (no separate zero fill or bias add).  A holds the
    // bias in k = 0..3 of lanes 0..31 (a 16-bit bias times 1.0 is exact), B of
    // tile column j holds 1.0 at k = j only, so each product picks the bias
    // once and the 16 MFMAs stay distinct.  (I8 starts from zero integers
    // and adds the bias the same way once its sums are scaled to fp32.)
    auto bias_mfma = [&](bool onto) {
      const bool lo = lane < 32;
      const unsigned one = lo ? (DT == SVDQ_BF16 ? 0x3F80u : 0x3C00u) : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned bh = lo ? (pack2<DT>(bcol[i], 0.0f) & 0xFFFFu) : 0u;
        const u32x4 ab = u32x4{bh | (bh << 16), bh | (bh << 16), 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 bj = u32x4{j == 0 ? one : j == 1 ? one << 16 : 0u, j == 2 ? one : j == 3 ? one << 16 : 0u, 0u, 0u};
          acc[i][j] = mfma32x16<DT>(ab, bj, onto ? acc[i][j] : f32x16{});
        }
      }
    };
    if constexpr (!I8) {
      // This wave's bias region holds its own loads only, so no barrier:
      // wait for the bias alone (every stage load was issued after it) and
      // run the bias MFMAs while the first stage lands.  (I8 reads the bias
      // after the K loop, so it is not live across it.)
      if (total > 3) SVDQ_WAIT_VM(4 * LPS);
      else if (total > 2) SVDQ_WAIT_VM(3 * LPS);
      else if (total > 1) SVDQ_WAIT_VM(2 * LPS);
      else SVDQ_WAIT_VM(LPS);
      read_bias();
      bias_mfma(false);
    }
    if (total > 3) SVDQ_WAIT_VM(3 * LPS);
    else if (total > 2) SVDQ_WAIT_VM(2 * LPS);
    else if (total > 1) SVDQ_WAIT_VM(LPS);
    else SVDQ_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    if constexpr (I8) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    }
    Frags F0, F1;
    read_frags(F0, 0);
    int r = 0;
    for (; r + 5 < nk; r += 2) {            // steady state: every step issued is a K step
      body_full(r, F0, F1);
      body_full(r + 1, F1, F0);
    }
    for (; r < nk; r += 2) {
      body_tail(r, F0, F1);
      if (r + 1 < nk) body_tail(r + 1, F1, F0);
    }
    if constexpr (I8) {
      // the exact int32 sums -> fp32 times s_x[m] s_w[n] (accumulator 4gg + x
      // of tile (i, j): column 32i + 8gg + 4(lane / 32) + x, token
      // 32j + lane % 32), then the bias; the low-rank steps add onto them
      const float* sxf = reinterpret_cast<const float*>(p.sx);
      const float* swf = reinterpret_cast<const float*>(p.sw);
      float sxv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sxv[j] = sxf[m0 + 128 * wm + 32 * j + (lane & 31)];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x16 swv;                              // s_w of this lane's 16 columns of tile i
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          int64_t nn = n0 + 128 * wn + 32 * i + 8 * gg + 4 * (lane >> 5);
          nn = nn + 4 <= p.N ? nn : p.N - 4;    // columns of a partial last tile are never stored
          const f32x4 sw = *reinterpret_cast<const f32x4*>(swf + nn);
#pragma unroll
          for (int x = 0; x < 4; ++x) swv[4 * gg + x] = sw[x];
        }
        // whole-vector conversion (the int32 sums are a bit-cast view of the accumulators)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_convertvector(__builtin_bit_cast(i32x16, acc[i][j]), f32x16) * (swv * sxv[j]);
      }
      read_bias();                           // the bias region of LDS is not part of the ring
      bias_mfma(true);
    }
    // low-rank steps (up to four were issued during the last K steps)
    for (int q = nk; q < total; ++q) {
      SVDQ_WAIT_LGKM0();
      SVDQ_WAIT_VM(0);
      __builtin_amdgcn_s_barrier();
      Frags F;
      read_frags(F, q & 3, false);
      if (q + 4 < total) {
        SVDQ_WAIT_LGKM0();
        __builtin_amdgcn_s_barrier();      // every wave has read step q
        issue(q + 4, q & 3);
      }
      // (otherwise the MFMAs wait for their own fragments only, so the
      // first ones start while the later reads are still in flight)
      compute_lr(q - nk, F);
    }
    SVDQ_WAIT_LGKM0();
    SVDQ_WAIT_VM(0);

    // ---- epilogue: (GELU,) round; stage the wave's 128 x 128 tile in LDS as
    // [token][column] rows, then store whole 256-byte row segments.  The
    // tile goes in two halves of 64 tokens: the second half's GELU and
    // staging run while the first half's stores drain.  Both halves stay
    // staged, so the chained epilogue below sees the whole tile.
    SVDQ_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();          // every wave is done with the LDS ring
    uint8_t* ob = smem + wave * (128 * mx::OUT_PITCH);
    const int64_t nw = n0 + 128 * wn;      // first column of this wave's tile
    const int64_t mw = m0 + 128 * wm;      // first token of this wave's tile
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          // accumulator 4gg + r of tile (i, j): column 32i + 8gg + 4(lane / 32) + r, token 32j + lane % 32
          const int nl = 32 * i + 8 * gg + 4 * (lane >> 5);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * hf + jj;
            float vv[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              vv[x] = acc[i][j][4 * gg + x];
              if constexpr (GELU) vv[x] = gelu_erf(vv[x]);
            }
            const int ml = 32 * j + (lane & 31);
            *reinterpret_cast<u32x2*>(ob + ml * mx::OUT_PITCH + nl * 2) = u32x2{pack2<DT>(vv[0], vv[1]), pack2<DT>(vv[2], vv[3])};
          }
        }
      }
      SVDQ_WAIT_LGKM0();
      if (nw < p.N && (!CHAIN || p.Y != nullptr)) {
        // non-temporal stores: Y is not read again here, and streaming it out
        // leaves fewer dirty lines for the next kernel's reads to wait behind;
        // the half's 16 row reads all issued ahead of their stores (forward
        // -1.4%, K2 -1.0% against four at a time, four interleaved rounds)
#pragma unroll
        for (int it = 16 * hf; it < 16 * hf + 16; ++it) {
          const int row = 4 * it + (lane >> 4);
          const int col = (lane & 15) * 8;
          const u32x4 val = *reinterpret_cast<const u32x4*>(ob + row * mx::OUT_PITCH + col * 2);
          if (mw + row < p.M)
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(p.Y + (mw + row) * p.ldy + nw + col));
        }
      }
    }
    if constexpr (CHAIN) chain_epilogue<DT>(p, smem, ob, wave, lane, m0, n0, nw, mw);
  }
  trace_mark(p.trace, 2);
}

// ---------------------------------------- k2_mx8 (MXFP4, two waves per SIMD)
// The MXFP4 GEMM with two waves on every SIMD, so one wave's LDS reads,
// waits and barrier stalls (and its epilogue) run under another's MFMAs.  A
// workgroup = WN x WM waves, each TI x TJ tiles of 32 x 32 on
// V_MFMA_SCALE_F32_32X32X64_F8F6F4; four-wave workgroups run two to a
// compute unit (the 192 x 192 tile in use), eight-wave ones alone.  A K step
// is taken in its two 64-deep halves: the MFMAs of one half run while the
// fragments of the other half (and of the next step) are read from LDS, so
// a wave holds one half-step of fragments twice over instead of a whole step
// twice over (144 accumulators and 48 fragment registers fit the 256 a wave
// has at two waves per SIMD).  Stages: a ring of K steps filled by buffer
// loads straight into LDS; after the per-step barrier the stage of the step
// just finished is refilled with the step STAGES ahead.  Every wave issues
// the same number of stage loads per step (so one immediate s_waitcnt count
// fits all waves): the fragment halves are dealt out first, then the e8m0
// pair dwords, the spare slots repeating the last pair.  The steady-state
// step has no branches (the compiler keeps the MFMA / memory interleave of
// a single basic block); the last steps, which may request low-rank steps,
// take a branchy path.  Bias, the low-rank up-projection and the epilogue
// (GELU, rounding, row-staged non-temporal stores) are as in k2_mx; the
// whole workgroup tile is staged at once.
namespace mx8 {
constexpr int scale_slots_low(int FR, int S, int NW) {
  int sl = 0;
  while (FR * sl + (NW - FR) * (sl + 1) < S) ++sl;
  return sl;
}
template <int WN_, int WM_, int TI_, int TJ_, int STAGES_ = 4>
struct Cfg {
  static constexpr int WN = WN_, WM = WM_, TI = TI_, TJ = TJ_;
  static constexpr int NW = WN * WM;                        // waves per workgroup
  static_assert(NW == 8 || NW == 4, "four or eight waves");
  static constexpr int NT = WN * TI, MT = WM * TJ;          // 32-row tiles of the workgroup tile
  static constexpr int TN = 32 * NT, TM = 32 * MT;
  static constexpr int NPA = (NT + 1) / 2, NPB = (MT + 1) / 2;   // e8m0 dword pairs per step
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = NT * 2048;
  static constexpr int SA_OFF = B_OFF + MT * 2048;
  static constexpr int SB_OFF = SA_OFF + NPA * 256;
  static constexpr int STAGE = SB_OFF + NPB * 256;
  static constexpr int STAGES = STAGES_;
  static_assert(STAGES == 3 || STAGES == 4, "stage ring");
  // workgroups per compute unit: eight-wave tiles fill a CU alone, four-wave
  // tiles run two to a CU (two waves per SIMD either way)
  static constexpr int WG_PER_CU = NW == 8 ? 1 : 2;
  // stage loads per step: F fragment halves (1 KB each), S pair dwords (256 B
  // each); waves below FR take FQ + 1 fragment halves and SL pairs, the
  // others FQ halves and SL + 1 pairs
  static constexpr int F = 2 * NT + 2 * MT, S = NPA + NPB;
  static constexpr int FQ = F / NW, FR = F % NW;
  static constexpr int SL = scale_slots_low(FR, S, NW);
  static constexpr int LPW = FQ + SL + 1;
  static constexpr int PITCH = TN * 2 + 16;                   // staged output row bytes
  static constexpr int LDS = STAGES * STAGE > TM * PITCH ? STAGES * STAGE : TM * PITCH;
};
// 192 x 192, two workgroups per compute unit (the one in use, for layers
// with a GELU epilogue: one workgroup's epilogue runs under the other's K
// loop); 384 x 192 and 256 x 256 eight-wave tiles were measured too
using Pair = Cfg<2, 2, 3, 3, 3>;
static_assert(Pair::LDS + Pair::NW * 512 <= 80 * 1024, "two workgroups per compute unit");
static_assert(Pair::FR == 0 && Pair::SL == 1 && Pair::LPW == 8, "load classes");
}  // namespace mx8

// One wave's share of a workgroup tile.  PA / PB: parity of the wave's first
// weight / token tile in the workgroup tile (it fixes where each tile's e8m0
// bytes sit in the pair dwords, byte 2 (tile % 2) + half); CLS: the wave's
// load class (0: one more fragment half, one pair dword fewer).
template <int DT, class C>
__device__ __forceinline__ void mx8_chain_epilogue(const MxParams& p, const uint8_t* smem, int wave, int lane,
                                                   int64_t n0, int64_t m0);

template <int DT, bool GELU, class C, int PA, int PB, int CLS, bool CHAIN = false>
__device__ __forceinline__ void mx8_tile(const MxParams& p, uint8_t* smem, int wave, int lane, int64_t n0, int64_t m0) {
  constexpr int TI = C::TI, TJ = C::TJ, LPW = C::LPW;
  constexpr int NF = CLS == 0 ? C::FQ + 1 : C::FQ;                         // fragment slots
  constexpr int NSA = (PA + TI - 1) / 2 + 1, NSB = (PB + TJ - 1) / 2 + 1;   // pair dwords read per side
  const int wn = wave % C::WN, wm = wave / C::WN;
  const int ia0 = wn * TI, jb0 = wm * TJ;              // first tile of the wave in the workgroup tile
  const int nsteps = int(p.K / KSTEP);
  const int64_t ntiles_n = p.N / 32;
  const int64_t ntiles_m = p.tiles_m_pad32;            // 32-row token tiles in the workspace
  const int cs = p.slots / 16;
  const int nk = nsteps;
  const int total = nk + (p.nchunks16 + 1) / 2;

  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)p.l2, 0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc((void*)p.xq, 0, -1, 0x00020000);
  const int lo16 = lane * 16, lo4 = lane * 4;

  // ---- this wave's stage loads (uniform): source offset of K step 0, source
  // offset of low-rank chunk 0 (fragment slots), LDS offset | half << 20 |
  // workspace-side << 21
  int src_k[LPW], src_lr[LPW], info[LPW];
  {
    const int f0 = CLS == 0 ? wave * (C::FQ + 1) : C::FR * (C::FQ + 1) + (wave - C::FR) * C::FQ;
    const int g0 = CLS == 0 ? wave * C::SL : C::FR * C::SL + (wave - C::FR) * (C::SL + 1);
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      if (k < NF) {
        const int u = f0 + k;
        if (u < 2 * C::NT) {
          const int t = u >> 1, h = u & 1;
          int64_t nt = n0 / 32 + t;
          nt = nt < ntiles_n ? nt : ntiles_n - 1;      // a partial last tile re-reads a valid tile
          src_k[k] = p.off_wq + int(nt * nsteps * 2 + h) * 1024;
          src_lr[k] = int(nt * cs) * 1024;
          info[k] = (C::A_OFF + u * 1024) | (h << 20);
        } else {
          const int v = u - 2 * C::NT, t = v >> 1, h = v & 1;
          int64_t mt = m0 / 32 + t;
          mt = mt < ntiles_m ? mt : ntiles_m - 1;
          src_k[k] = int(mt * nsteps * 2 + h) * 1024;
          src_lr[k] = p.off_t + int(mt * cs) * 1024;
          info[k] = (C::B_OFF + v * 1024) | (h << 20) | (1 << 21);
        }
      } else {
        int g = g0 + (k - NF);
        g = g < C::S ? g : C::S - 1;                   // the spare slots repeat the last pair
        if (g < C::NPA) {
          int64_t pn = n0 / 64 + g;
          pn = pn < p.N / 64 ? pn : p.N / 64 - 1;
          src_k[k] = p.off_sw + int(pn * nsteps) * 256;
          info[k] = C::SA_OFF + g * 256;
        } else {
          const int q = g - C::NPA;
          int64_t pm = m0 / 64 + q;
          pm = pm < ntiles_m / 2 ? pm : ntiles_m / 2 - 1;
          src_k[k] = p.off_sx + int(pm * nsteps) * 256;
          info[k] = (C::SB_OFF + q * 256) | (1 << 21);
        }
        src_lr[k] = src_k[k];
      }
    }
  }
  // slot k of K step r into stage r % 4
  auto issue_k = [&](int r, int k) {
    uint8_t* base = smem + (r % C::STAGES) * C::STAGE + (info[k] & 0xFFFFF);
    const __amdgpu_buffer_rsrc_t rs = (info[k] & (1 << 21)) ? rsw : rsb;
    if (k < NF) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)base, 16, lo16, src_k[k] + r * 2048, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)base, 4, lo4, src_k[k] + r * 256, 0, 0);
  };
  // slot k of step r, a K step or a low-rank step (chunks 2e, 2e + 1 of L2
  // and T in the fragment slots; the pair slots reload K step 0's)
  auto issue_any = [&](int r, int k) {
    if (r < nk) {
      issue_k(r, k);
      return;
    }
    uint8_t* base = smem + (r % C::STAGES) * C::STAGE + (info[k] & 0xFFFFF);
    const __amdgpu_buffer_rsrc_t rs = (info[k] & (1 << 21)) ? rsw : rsb;
    if (k < NF) {
      int c = 2 * (r - nk) + ((info[k] >> 20) & 1);
      c = c < p.nchunks16 ? c : p.nchunks16 - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)base, 16, lo16, src_lr[k] + c * 1024, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)base, 4, lo4, src_lr[k], 0, 0);
    }
  };

  // ---- fragments: one half-step of each side, twice (halves 0 and 1)
  u32x4 fa[2][TI], fb[2][TJ];
  unsigned sa[NSA], sb[NSB], na[NSA], nb[NSB];      // e8m0 pair dwords: current / next step
  auto rd_a = [&](int st, int h, int i) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(smem + st * C::STAGE + C::A_OFF + ((ia0 + i) * 2 + h) * 1024 + lo16);
  };
  auto rd_b = [&](int st, int h, int j) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(smem + st * C::STAGE + C::B_OFF + ((jb0 + j) * 2 + h) * 1024 + lo16);
  };
  auto rd_sa = [&](int st, int d) -> unsigned {
    int q = ia0 / 2 + d;
    q = q < C::NPA ? q : C::NPA - 1;
    return *reinterpret_cast<const unsigned*>(smem + st * C::STAGE + C::SA_OFF + q * 256 + lo4);
  };
  auto rd_sb = [&](int st, int d) -> unsigned {
    int q = jb0 / 2 + d;
    q = q < C::NPB ? q : C::NPB - 1;
    return *reinterpret_cast<const unsigned*>(smem + st * C::STAGE + C::SB_OFF + q * 256 + lo4);
  };
  // read x of the next step's half 0: fragments, then pair dwords
  constexpr int NRD = TI + TJ + NSA + NSB;
  auto rd_next = [&](int st, int x) {
    if (x < TI) fa[0][x] = rd_a(st, 0, x);
    else if (x < TI + TJ) fb[0][x - TI] = rd_b(st, 0, x - TI);
    else if (x < TI + TJ + NSA) na[x - TI - TJ] = rd_sa(st, x - TI - TJ);
    else nb[x - TI - TJ - NSA] = rd_sb(st, x - TI - TJ - NSA);
  };

  f32x16 acc[TI][TJ];
  // MFMA (h, i, j) with the e8m0 bytes of tile i / j picked by op_sel
  auto mfma_hij = [&](int h, int i, int j) {
    const u32x4 av = fa[h][i], bv = fb[h][j];
    const i32x8 a = i32x8{int(av[0]), int(av[1]), int(av[2]), int(av[3]), 0, 0, 0, 0};
    const i32x8 b = i32x8{int(bv[0]), int(bv[1]), int(bv[2]), int(bv[3]), 0, 0, 0, 0};
    acc[i][j] = mfma_mx32(a, b, acc[i][j], int(sa[(PA + i) / 2]), int(sb[(PB + j) / 2]), 2 * ((PA + i) & 1) + h,
                          2 * ((PB + j) & 1) + h);
  };

  // ---- prologue: bias of this wave's columns (to LDS by buffer loads, as
  // in k2_mx, so only the first stage is waited for), the first stages
  static_assert(TI * 32 <= 128, "a wave's bias values fit its 512 bytes");
  float* bias_lds = reinterpret_cast<float*>(smem + C::LDS + wave * 512);
  {
    const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc((void*)p.bias, 0, -1, 0x00020000);
#pragma unroll
    for (int h = 0; h < (TI * 32 + 63) / 64; ++h) {
      int64_t nb_ = n0 + 32 * ia0 + 64 * h + lane;
      nb_ = nb_ < p.N ? nb_ : p.N - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rbias, (lds_ptr_t)(bias_lds + 64 * h), 4, int(nb_) * 4, 0, 0, 0);
    }
  }
  for (int r = 0; r < C::STAGES && r < total; ++r) {
#pragma unroll
    for (int k = 0; k < LPW; ++k) issue_any(r, k);
  }
  // this wave's bias region holds its own loads only: wait for the bias
  // alone (every stage load was issued after it), so the bias MFMAs run
  // while the first stage lands
  if (C::STAGES > 3 && total > 3) SVDQ_WAIT_VM(4 * LPW);
  else if (total > 2) SVDQ_WAIT_VM(3 * LPW);
  else if (total > 1) SVDQ_WAIT_VM(2 * LPW);
  else SVDQ_WAIT_VM(LPW);
  float bcol[TI];
#pragma unroll
  for (int i = 0; i < TI; ++i) bcol[i] = bias_lds[32 * i + (lane & 31)];
  {
    // accumulators start at the bias (see k2_mx)
    const bool lo = lane < 32;
    const unsigned one = lo ? (DT == SVDQ_BF16 ? 0x3F80u : 0x3C00u) : 0u;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const unsigned bh = lo ? (pack2<DT>(bcol[i], 0.0f) & 0xFFFFu) : 0u;
      const u32x4 ab = u32x4{bh | (bh << 16), bh | (bh << 16), 0u, 0u};
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int jj = j & 3;
        const u32x4 bj = u32x4{jj == 0 ? one : jj == 1 ? one << 16 : 0u, jj == 2 ? one : jj == 3 ? one << 16 : 0u, 0u, 0u};
        acc[i][j] = mfma32x16<DT>(ab, bj, f32x16{});
      }
    }
  }
  if (C::STAGES > 3 && total > 3) SVDQ_WAIT_VM(3 * LPW);
  else if (total > 2) SVDQ_WAIT_VM(2 * LPW);
  else if (total > 1) SVDQ_WAIT_VM(LPW);
  else SVDQ_WAIT_VM(0);
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int x = 0; x < NRD; ++x) rd_next(0, x);
#pragma unroll
  for (int d = 0; d < NSA; ++d) sa[d] = na[d];
#pragma unroll
  for (int d = 0; d < NSB; ++d) sb[d] = nb[d];

  // ---- K steps.  Step r:
  //  phase A: the half-0 MFMAs, with the half-1 fragments of step r read in
  //           between;
  //  phase B: wait for step r + 1 (own loads, then the barrier for all
  //           waves'), then the half-1 MFMAs with the half-0 fragments and
  //           pair dwords of step r + 1 read in between, and step r's stage
  //           refilled with the step STAGES ahead.
  auto phase_a = [&](int r) {
    const int st = r % C::STAGES;
    SVDQ_WAIT_LGKM0();
#pragma unroll
    for (int k = 0; k < TI * TJ; ++k) {
      mfma_hij(0, k / TJ, k % TJ);
      if (k < TI) fa[1][k] = rd_a(st, 1, k);
      else if (k < TI + TJ) fb[1][k - TI] = rd_b(st, 1, k - TI);
      __builtin_amdgcn_sched_barrier(0);
    }
    SVDQ_WAIT_LGKM0();
  };
  auto commit_scales = [&]() {
#pragma unroll
    for (int d = 0; d < NSA; ++d) sa[d] = na[d];
#pragma unroll
    for (int d = 0; d < NSB; ++d) sb[d] = nb[d];
  };
  // steady state (r + STAGES < nk): no branches, the memory operations of
  // phase B two per MFMA (the reads first, the stage refill after)
  constexpr int AHEAD = C::STAGES;
  auto kstep = [&](int r) {
    phase_a(r);
    SVDQ_WAIT_VM((C::STAGES - 2) * LPW);
    __builtin_amdgcn_s_barrier();
    const int st1 = (r + 1) % C::STAGES;
#pragma unroll
    for (int k = 0; k < TI * TJ; ++k) {
      mfma_hij(1, k / TJ, k % TJ);
#pragma unroll
      for (int x = 2 * k; x < 2 * k + 2; ++x) {
        if (x < NRD) rd_next(st1, x);
        else if (x - NRD < LPW) issue_k(r + AHEAD, x - NRD);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int x = 2 * TI * TJ; x < NRD + LPW; ++x) {
      if (x < NRD) rd_next(st1, x);
      else issue_k(r + AHEAD, x - NRD);
    }
    __builtin_amdgcn_sched_barrier(0);
    commit_scales();
  };
  // the last K steps: waits, refills (possibly low-rank steps) and reads
  // under branches, then the half-1 MFMAs
  auto kstep_tail = [&](int r) {
    phase_a(r);
    if (r + 1 < total) {
      // steps after r + 1 already requested: r + 2 .. r + STAGES - 1, those that exist
      if (C::STAGES > 3 && r + 3 < total) SVDQ_WAIT_VM(2 * LPW);
      else if (r + 2 < total) SVDQ_WAIT_VM(LPW);
      else SVDQ_WAIT_VM(0);
      __builtin_amdgcn_s_barrier();
    }
    if (r + AHEAD < total) {
#pragma unroll
      for (int k = 0; k < LPW; ++k) issue_any(r + AHEAD, k);
    }
    if (r + 1 < nk) {
#pragma unroll
      for (int x = 0; x < NRD; ++x) rd_next((r + 1) % C::STAGES, x);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < TI * TJ; ++k) mfma_hij(1, k / TJ, k % TJ);
    __builtin_amdgcn_sched_barrier(0);
    commit_scales();
  };
  int r = 0;
  for (; r + AHEAD < nk; ++r) kstep(r);
  for (; r < nk; ++r) kstep_tail(r);

  // ---- low-rank steps: T L2 on the 32 x 32 x 16 16-bit MFMA (the stage of
  // step q was waited for by the previous barrier)
  for (int q = nk; q < total; ++q) {
    SVDQ_WAIT_LGKM0();
    if (q > nk) {
      SVDQ_WAIT_VM(0);
      __builtin_amdgcn_s_barrier();
    }
    const int st = q % C::STAGES;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < TI; ++i) fa[h][i] = rd_a(st, h, i);
#pragma unroll
      for (int j = 0; j < TJ; ++j) fb[h][j] = rd_b(st, h, j);
    }
    if (q + AHEAD < total) {
      SVDQ_WAIT_LGKM0();
      __builtin_amdgcn_s_barrier();      // every wave has read stage q before it is refilled
#pragma unroll
      for (int k = 0; k < LPW; ++k) issue_any(q + AHEAD, k);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (2 * (q - nk) + h < p.nchunks16) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32x16<DT>(fa[h][i], fb[h][j], acc[i][j]);
      }
  }
  SVDQ_WAIT_LGKM0();
  SVDQ_WAIT_VM(0);
  __builtin_amdgcn_s_barrier();          // every wave is done with the ring

  // ---- epilogue: (GELU,) round; stage the workgroup tile in LDS as
  // [token][column] rows, then store whole row segments
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      // accumulator 4gg + x of tile (i, j): column 32i + 8gg + 4(lane / 32) + x, token 32j + lane % 32
      const int nl = 32 * (ia0 + i) + 8 * gg + 4 * (lane >> 5);
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        float vv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          vv[x] = acc[i][j][4 * gg + x];
          if constexpr (GELU) vv[x] = gelu_erf(vv[x]);
        }
        const int ml = 32 * (jb0 + j) + (lane & 31);
        *reinterpret_cast<u32x2*>(smem + ml * C::PITCH + nl * 2) = u32x2{pack2<DT>(vv[0], vv[1]), pack2<DT>(vv[2], vv[3])};
      }
    }
  }
  SVDQ_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  // 16-byte pieces of the staged rows: piece c of row t covers columns 8c .. 8c + 7
  constexpr int PPR = C::TN / 8;                       // pieces per row
  constexpr int NPC = C::TM * PPR;                     // pieces in the tile
  const int tid = wave * 64 + lane;
#pragma unroll 2
  for (int pc = tid; pc < NPC; pc += 64 * C::NW) {
    const int row = pc / PPR, c = pc % PPR;
    const u32x4 val = *reinterpret_cast<const u32x4*>(smem + row * C::PITCH + c * 16);
    if (m0 + row < p.M && n0 + 8 * c < p.N && (!CHAIN || p.Y != nullptr))
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(p.Y + (m0 + row) * p.ldy + n0 + 8 * c));
  }
  if constexpr (CHAIN) mx8_chain_epilogue<DT, C>(p, smem, wave, lane, n0, m0);
}

// Epilogue chaining on the paired tiles: the staged TM x TN tile (rounded,
// after GELU: the bits this layer would store) is the next layer's input
// over columns n0 .. n0 + TN.  Codes and scales: unit (token tile t of 32
// rows, 32-column block b) is one half-wave, lane = token row, applying the
// activation kernel's MXFP4 rule and writing one 16-byte fragment piece and
// one scale byte of the next layer's workspace (a 192-column tile covers
// one and a half 128-deep steps of the next layer, so scale bytes, not
// dwords, are stored).  Down-projection: each wave takes three 16-token
// groups and, for every next-layer step the tile touches, runs the
// 16 x 16 x 32 MFMAs with the step's L1x fragments, lanes whose k lies
// outside the tile contributing zero, into this tile's fp32 partial slab.
template <int DT, class C>
__device__ __forceinline__ void mx8_chain_epilogue(const MxParams& p, const uint8_t* smem, int wave, int lane,
                                                   int64_t n0, int64_t m0) {
  const int nst = int(p.N / KSTEP);                       // K steps of the next layer
  const int64_t ntok32 = p.tiles_m_pad32;                 // 32-row token tiles in the next workspace
  constexpr int TT = C::TM / 32, TB = C::TN / 32, NU = TT * TB;
  constexpr int NIT = (NU + 2 * C::NW - 1) / (2 * C::NW); // unit rounds per wave
  const int half = lane >> 5, r32 = lane & 31;
  // a unit's 1/lambda (32 columns) is requested one unit ahead
  f32x4 il[2][8];
  auto load_il = [&](int u, f32x4 (&dst)[8]) {
    int64_t col = n0 + 32 * (u % TB);
    col = (u < NU && col < p.N) ? col : 0;                // padding units read column 0 and store nothing
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = *reinterpret_cast<const f32x4*>(p.nx_invlam + col + 4 * e);
  };
  load_il(2 * wave + half, il[0]);
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int u = 2 * wave + 2 * C::NW * k + half, t = u / TB, b = u % TB;
    if (k + 1 < NIT) load_il(u + 2 * C::NW, il[(k + 1) & 1]);
    const int64_t col = n0 + 32 * b;
    const int64_t tg = m0 / 32 + t;
    if (u < NU && col < p.N && tg < ntok32) {
      const f32x4 (&ilk)[8] = il[k & 1];
      const uint8_t* src = smem + (32 * t + r32) * C::PITCH + 64 * b;
      float xh[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + 16 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = 8 * i + 2 * e;
          xh[x] = h2f<DT>(v[e] & 0xFFFFu) * ilk[x >> 2][x & 3];
          xh[x + 1] = h2f<DT>(v[e] >> 16) * ilk[(x + 1) >> 2][(x + 1) & 3];
        }
      }
      float am = 0.0f;
#pragma unroll
      for (int x = 0; x < 32; ++x) am = fmaxf(am, fabsf(xh[x]));
      const int ex = e8m0_needs_slow(am) ? e8m0_slow(am) : e8m0_fast(am);
      const float scl = ex != 0 ? __uint_as_float(unsigned(ex) << 23) : 1.0f;
      unsigned d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        unsigned v = 0u;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const unsigned cv = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, xh[8 * i + 2 * bb], xh[8 * i + 2 * bb + 1], scl, 0);
          v |= (cv & 0xFFu) << (8 * bb);
        }
        d[i] = v;
      }
      const int s2 = int(col / KSTEP), bis = int((col % KSTEP) / 32);   // next-layer step, block in the step
      *reinterpret_cast<u32x4*>(p.nx_xq + ((size_t(tg) * nst + s2) * 2 + (bis >> 1)) * 1024 + (r32 + 32 * (bis & 1)) * 16) =
          u32x4{d[0], d[1], d[2], d[3]};
      p.nx_sx[((size_t(tg >> 1) * nst + s2) * 64 + r32 + 32 * (bis & 1)) * 4 + 2 * (tg & 1) + (bis >> 1)] = uint8_t(ex);
    }
  }
  if (p.nx_njt == 0) return;
  // down-projection partials of this column tile: the tile's staged values
  // are read once (two next-layer steps x four MFMA k slices x the wave's
  // 16-token groups) and reused for every 16-rank chunk; the L1x fragments
  // of chunk jt + 1 are requested while chunk jt's MFMAs run
  const int cs = p.nx_slots / 16;
  const int q = lane >> 4;
  const int64_t ncol = (n0 + C::TN < p.N ? n0 + C::TN : p.N);    // end of the tile's columns
  const int s_first = int(n0 / KSTEP);
  // next-layer steps a tile can touch (tiles start at multiples of 64 columns)
  constexpr int NS = (C::TN + 64 + KSTEP - 1) / KSTEP;
  static_assert(C::TN % 64 == 0, "tiles start at multiples of 64 columns");
  constexpr int NG = C::TM / 16;                                  // 16-token groups of the tile
  constexpr int GPW = (NG + C::NW - 1) / C::NW;                   // per wave
  const u32x4* l1x = reinterpret_cast<const u32x4*>(p.nx_l1x);
  u32x4 xv[NS][4][GPW];
#pragma unroll
  for (int sv = 0; sv < NS; ++sv)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // MFMA c takes k in [32q + 8c, +8) of step s_first + sv from lane group q
      const int64_t k = int64_t(s_first + sv) * KSTEP + 32 * q + 8 * c;
      const bool in = k >= n0 && k < ncol;
      const int off = in ? int(k - n0) * 2 : 0;
#pragma unroll
      for (int g = 0; g < GPW; ++g) {
        const int grp = wave + C::NW * g;
        const u32x4 v = grp < NG ? *reinterpret_cast<const u32x4*>(smem + (16 * grp + (lane & 15)) * C::PITCH + off)
                                 : u32x4{0u, 0u, 0u, 0u};
        xv[sv][c][g] = in ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  const int s_max = nst - 1;
  u32x4 la[2][NS][4];
  auto load_la = [&](int jt, u32x4 (&dst)[NS][4]) {
#pragma unroll
    for (int sv = 0; sv < NS; ++sv) {
      const int s2 = s_first + sv <= s_max ? s_first + sv : s_max;   // a step past the layer reads the last (its lanes are zero)
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[sv][c] = l1x[((size_t(s2) * cs + jt) * 4 + c) * 64 + lane];
    }
  };
  float* tp = p.nx_tp + (size_t(n0 / C::TN) * p.nx_Mp + m0) * p.nx_slots;
  load_la(0, la[0]);
  for (int jt = 0; jt < p.nx_njt; jt += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = jt + h;
      if (j < p.nx_njt) {
        if (j + 1 < p.nx_njt) load_la(j + 1, la[h ^ 1]);
        f32x4 acc[GPW];
#pragma unroll
        for (int g = 0; g < GPW; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sv = 0; sv < NS; ++sv)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int g = 0; g < GPW; ++g) acc[g] = mfma16<DT>(la[h][sv][c], xv[sv][c][g], acc[g]);
        // lane holds T[token 16 grp + lane % 16][16 j + 4 q + i]
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
          const int grp = wave + C::NW * g;
          const int64_t row = m0 + 16 * grp + (lane & 15);
          if (grp < NG && row < p.nx_Mp)
            *reinterpret_cast<f32x4*>(tp + size_t(16 * grp + (lane & 15)) * p.nx_slots + 16 * j + 4 * q) = acc[g];
        }
      }
    }
  }
}

template <int DT, bool GELU, class C, bool CHAIN = false>
__global__ __launch_bounds__(64 * C::NW, C::WG_PER_CU) void k2_mx8(MxParams p) {
  trace_mark(p.trace, 0);
  stagger_start(p.stagger_wgs, p.stagger_sleeps);
  // (the ring / output staging, then each wave's bias values)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS + C::NW * 512];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // XCD-aware grouped tile order (as in k2_mx)
  const int T = p.tiles_n * p.tiles_m;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, kx = bid >> 3, per = T >> 3, rem = T & 7;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int gsz_full = mx::GROUP_M * p.tiles_n;
  const int grp = tile / gsz_full, first_m = grp * mx::GROUP_M;
  const int gm = (p.tiles_m - first_m) < mx::GROUP_M ? (p.tiles_m - first_m) : mx::GROUP_M;
  const int within = tile - grp * gsz_full;
  const int tm = first_m + within % gm, tn = within / gm;
  const int64_t n0 = int64_t(tn) * C::TN, m0 = int64_t(tm) * C::TM;
  const int pa = ((wave % C::WN) * C::TI) & 1, pb = ((wave / C::WN) * C::TJ) & 1;
  // one load class (every wave issues the same stage loads), four tile parities
  static_assert(C::FR == 0, "one load class");
  if (pb == 0) {
    if (pa == 0) mx8_tile<DT, GELU, C, 0, 0, 1, CHAIN>(p, smem, wave, lane, n0, m0);
    else mx8_tile<DT, GELU, C, 1, 0, 1, CHAIN>(p, smem, wave, lane, n0, m0);
  } else {
    if (pa == 0) mx8_tile<DT, GELU, C, 0, 1, 1, CHAIN>(p, smem, wave, lane, n0, m0);
    else mx8_tile<DT, GELU, C, 1, 1, 1, CHAIN>(p, smem, wave, lane, n0, m0);
  }
  trace_mark(p.trace, 2);
}

// ------------------------------------------- unfused low-rank up-projection
// The unfused low-rank baseline's last pass: Y = round16(GELU?(Y + T L2)),
// reading and rewriting the 4-bit GEMM's rounded output.  Same fragment
// layouts and 16-bit MFMAs as the GEMM's fused low-rank steps: MXFP4
// layers use 32 x 32 x 16 tiles and 16-rank chunks, INT4 layers
// 16 x 16 x 32 tiles and 32-rank chunks.
struct UpParams {
  const uint16_t* l2;
  const uint16_t* t;
  uint16_t* Y;
  int64_t ldy, M, N;
  int slots, nchunks;    // rank slots; MFMA K chunks of the active rank
};

// A wave owns ROWS tokens x 128 columns.  Its Y rows are loaded first, as
// 16-byte pieces of whole rows (16 lanes per 256-byte row piece), so the
// loads run under the MFMAs; the fp32 products then go through LDS into the
// same row order, and each lane adds, rounds and stores its pieces.
template <int DT, int FMT, bool GELU>
__global__ __launch_bounds__(256) void k_up(UpParams p) {
  constexpr bool MX = FMT == SVDQ_FMT_MXFP4_G32;
  constexpr int ROWS = MX ? 32 : 16;             // tokens per wave
  constexpr int PITCH = 128 * 4 + 16;            // bytes per staged fp32 row
  constexpr int PIECES = ROWS * 16 / 64;         // 16-byte Y pieces per lane
  __shared__ __attribute__((aligned(16))) uint8_t stage[4 * ROWS * PITCH];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t n0 = int64_t(blockIdx.x) * 128;
  const int64_t m0 = int64_t(blockIdx.y) * (4 * ROWS) + ROWS * wave;
  if (m0 >= p.M) return;
  uint8_t* st = stage + wave * ROWS * PITCH;
  // Y pieces: piece c = 64 it + lane is row c / 16, columns 8 (c % 16) .. +8
  u32x4 y[PIECES];
#pragma unroll
  for (int it = 0; it < PIECES; ++it) {
    const int c = 64 * it + lane, row = c >> 4, col = (c & 15) * 8;
    y[it] = m0 + row < p.M ? *reinterpret_cast<const u32x4*>(p.Y + (m0 + row) * p.ldy + n0 + col)
                           : u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (MX) {
    // 4 tiles of 32 x 32 x 16, 16-rank chunks
    const int cs = p.slots / 16;
    const u32x4* tb = reinterpret_cast<const u32x4*>(p.t) + (m0 / 32) * cs * 64 + lane;
    const u32x4* lb = reinterpret_cast<const u32x4*>(p.l2) + (n0 / 32) * cs * 64 + lane;
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
    for (int c = 0; c < p.nchunks; ++c) {
      const u32x4 b = tb[c * 64];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = mfma32x16<DT>(lb[(i * cs + c) * 64], b, acc[i]);
    }
    // accumulator 4gg + x of tile i: column 32i + 8gg + 4(lane / 32) + x, token lane % 32
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *reinterpret_cast<f32x4*>(st + (lane & 31) * PITCH + (32 * i + 8 * gg + 4 * (lane >> 5)) * 4) =
            f32x4{acc[i][4 * gg], acc[i][4 * gg + 1], acc[i][4 * gg + 2], acc[i][4 * gg + 3]};
  } else {
    // 8 tiles of 16 x 16 x 32, 32-rank chunks
    const int cs = p.slots / 32;
    const u32x4* tb = reinterpret_cast<const u32x4*>(p.t) + (m0 / 16) * cs * 64 + lane;
    const u32x4* lb = reinterpret_cast<const u32x4*>(p.l2) + (n0 / 16) * cs * 64 + lane;
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < p.nchunks; ++c) {
      const u32x4 b = tb[c * 64];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = mfma16<DT>(lb[(i * cs + c) * 64], b, acc[i]);
    }
    // accumulator x of tile i: column 16i + 4(lane / 16) + x, token lane % 16
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<f32x4*>(st + (lane & 15) * PITCH + (16 * i + 4 * (lane >> 4)) * 4) = acc[i];
  }
  SVDQ_WAIT_LGKM0();                 // the wave reads back only its own rows
#pragma unroll
  for (int it = 0; it < PIECES; ++it) {
    const int c = 64 * it + lane, row = c >> 4, col = (c & 15) * 8;
    if (m0 + row >= p.M) continue;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(st + row * PITCH + col * 4);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(st + row * PITCH + col * 4 + 16);
    float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    unsigned o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float lo = h2f<DT>(y[it][e] & 0xFFFFu) + v[2 * e], hi = h2f<DT>(y[it][e] >> 16) + v[2 * e + 1];
      if constexpr (GELU) {
        lo = gelu_erf(lo);
        hi = gelu_erf(hi);
      }
      o[e] = pack2<DT>(lo, hi);
    }
    *reinterpret_cast<u32x4*>(p.Y + (m0 + row) * p.ldy + n0 + col) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

// -------------------------------------------------- INT4 per-group products
// Finishes a chained down-projection: T[m][j] = round16(sum over the
// column-tile slabs of the fp32 partials), written in the GEMM's low-rank
// operand layout.  A workgroup covers 64 (token, 4-rank) items; its four
// waves each sum a fixed quarter of the slabs and wave 0 adds the quarters
// in order, so the result does not depend on scheduling.
struct TfinParams {
  const float* tp;       // [nparts][Mp][slots]
  uint16_t* t;
  int64_t Mp;
  int slots, nparts, ncols4;
};

template <int DT, int FMT>
__global__ __launch_bounds__(256) void k_tfin(TfinParams p) {
  __shared__ f32x4 part[3][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t g = int64_t(blockIdx.x) * 64 + lane;
  const int64_t m = g / p.ncols4;
  const int j4 = int(g % p.ncols4);
  const bool ok = m < p.Mp;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ok) {
    const float* src = p.tp + m * p.slots + 4 * j4;
    const size_t stride = size_t(p.Mp) * size_t(p.slots);
    const int q0 = (p.nparts * w) / 4, q1 = (p.nparts * (w + 1)) / 4;
#pragma unroll 4
    for (int q = q0; q < q1; ++q) s += *reinterpret_cast<const f32x4*>(src + q * stride);
  }
  if (w > 0) part[w - 1][lane] = s;
  __syncthreads();
  if (w == 0 && ok) {
    s += part[0][lane];
    s += part[1][lane];
    s += part[2][lane];
    const int j = 4 * j4;
    uint16_t* dst;
    if constexpr (FMT == SVDQ_FMT_MXFP4_G32) {
      // MXFP4 low-rank layout: 32-row tiles, 16-rank chunks, lane (row % 32) + 32 (j % 16 >= 8)
      const int c = j / 16, jj = j % 16;
      const int64_t ln = (m % 32) + 32 * (jj / 8);
      dst = p.t + (((m / 32) * (p.slots / 16) + c) * 64 + ln) * 8 + (jj % 8);
    } else {
      // INT4 low-rank layout: 16-row tiles, 32-rank chunks; the activation
      // kernel's lane (m, q) of 16-rank tile jt holds ranks 16 jt + 4q .. + 3
      const int jt = j / 16, q = (j % 16) / 4;
      const int64_t ln = (m % 16) + 16 * (2 * (jt & 1) + (q >> 1));
      dst = p.t + (((m / 16) * (p.slots / 32) + (jt >> 1)) * 64 + ln) * 8 + 4 * (q & 1);
    }
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack2<DT>(s[0], s[1]), pack2<DT>(s[2], s[3])};
  }
}

struct PartialParams {
  const uint8_t* wq;
  const uint8_t* xq;
  int32_t* out;
  int64_t K, m0, nm, n0, nn, g0;
};

// One wave per (16 n, 16 m, group): the same fragments and integer MFMA as
// k2_gemm, written out instead of dequantized.
__global__ __launch_bounds__(64) void k_int4_partials(PartialParams p) {
  const int lane = threadIdx.x;
  const int q = lane >> 4;
  const int64_t nt = (p.n0 / 16) + blockIdx.x, mt = (p.m0 / 16) + blockIdx.y;
  const int64_t G = p.g0 + blockIdx.z;
  const int nsteps = int(p.K / KSTEP);
  const int64_t s = G / 2;
  const int g = int(G % 2);
  const u32x4 a = reinterpret_cast<const u32x4*>(p.wq)[(nt * nsteps + s) * 64 + lane];
  const u32x4 b = reinterpret_cast<const u32x4*>(p.xq)[(mt * nsteps + s) * 64 + lane];
  const i32x4 P = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_nibbles(a[2 * g], a[2 * g + 1]),
                                                       widen_nibbles(b[2 * g], b[2 * g + 1]), i32x4{0, 0, 0, 0}, 0, 0, 0);
  const int64_t mm = int64_t(blockIdx.y) * 16 + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t nn = int64_t(blockIdx.x) * 16 + 4 * q + r;
    p.out[(int64_t(blockIdx.z) * p.nm + mm) * p.nn + nn] = P[r] >> 8;   // operands carry 16*q each
  }
}

// --------------------------------------------------- calibration statistic
template <int DT>
__global__ __launch_bounds__(256) void k_absmax(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                                int64_t rows_per_block, float* absmax) {
  const int64_t k = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (k >= K) return;
  const int64_t r0 = int64_t(blockIdx.y) * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < M ? r0 + rows_per_block : M;
  float m = 0.0f;
  for (int64_t r = r0; r < r1; ++r) m = fmaxf(m, fabsf(h2f<DT>(X[r * ldx + k])));
  // non-negative floats order like their bit patterns
  atomicMax(reinterpret_cast<unsigned*>(absmax) + k, __float_as_uint(m));
}

inline svdq_status launch_ok() { return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP; }

// Kernel timing (svdq_timing_start / svdq_timing_stop): while it is on for a
// host thread, that thread's activation-kernel, GEMM and low-rank-pass
// launches go through hipExtLaunchKernel with an event pair of their own,
// which takes the kernel's own dispatch begin / end timestamps -- nothing is
// added to the stream between kernels.
struct KernelTiming {
  bool on = false;
  std::vector<hipEvent_t> ev;   // begin, end per launch slot
  std::vector<int> kind;        // svdq_kernel_kind of the launch in each used slot
  size_t used = 0;
};
thread_local KernelTiming t_timing;

template <typename F, typename... A>
void launch(svdq_kernel_kind kind, F kernel, dim3 grid, dim3 block, unsigned lds, hipStream_t st, A... args) {
  KernelTiming& t = t_timing;
  if (t.on && t.used < t.kind.size()) {
    hipEvent_t b = t.ev[2 * t.used], e = t.ev[2 * t.used + 1];
    t.kind[t.used++] = int(kind);
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, b, e, 0u, args...);
  } else {
    void* a[] = {static_cast<void*>(&args)...};
    (void)hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, a, lds, st);
  }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// compute units of the current device (queried once per device)
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int FMT, int DT, bool CHUNK, int TT = 1>
void launch_k1_as(const K1Params& kp, int64_t Mp, hipStream_t st) {
  const dim3 grid(unsigned(Mp / (16 * TT))), block(256);
  const bool il = kp.K <= K1_IL_LDS_MAX_K;
  const size_t il_bytes = il ? size_t((kp.K + 255) & ~int64_t(255)) * 4 : 0;
  auto red_bytes = [](int njt) { return size_t(TT) * (size_t(4) * size_t(njt) * 64 * 16 + K1_XBUF_BYTES); };
  if (kp.njt == 0) {
    if (il) launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, 0, true, true, CHUNK, TT>), grid, block, il_bytes + red_bytes(0), st, kp);
    else launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, 0, false, true, CHUNK, TT>), grid, block, red_bytes(0), st, kp);
  } else if (kp.njt <= 2) {
    if (il) launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, 2, true, true, CHUNK, TT>), grid, block, il_bytes + red_bytes(2), st, kp);
    else launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, 2, false, true, CHUNK, TT>), grid, block, red_bytes(2), st, kp);
  } else if (kp.njt <= 4) {
    if (il) launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, 4, true, true, CHUNK, TT>), grid, block, il_bytes + red_bytes(4), st, kp);
    else launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, 4, false, true, CHUNK, TT>), grid, block, red_bytes(4), st, kp);
  } else if constexpr (TT == 1) {   // (ranks above 64 keep one tile per workgroup)
    if (il) launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, MAXJT, true, true, CHUNK>), grid, block, il_bytes + red_bytes(MAXJT), st, kp);
    else launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, MAXJT, false, true, CHUNK>), grid, block, red_bytes(MAXJT), st, kp);
  }
}

template <int FMT, int DT>
void launch_k1(const K1Params& kp, int64_t Mp, hipStream_t st) {
  const int64_t tiles = Mp / 16, cus = int64_t(device_cus());
  if constexpr (FMT == SVDQ_FMT_MXFP4_G32) {
    // MXFP4 requests whole chunks of steps once more than two workgroups
    // per compute unit queue up
    if (tiles > 2 * cus) {
      launch_k1_as<FMT, DT, true>(kp, Mp, st);
      return;
    }
    // More 16-token tiles than compute units and a long K: two tiles per
    // workgroup, so each step's L1x fragments (twice the step's X bytes at
    // rank 32, read from L2) serve 32 tokens; one workgroup reading L1x
    // once for two tiles beats two workgroups on one compute unit reading
    // it twice (FLUX fc2, K = 12288: 55.5 -> 49.0 us).  At K = 3072 the two
    // forms take the same time.  INT4 keeps one tile per workgroup: its
    // heavier quantizer would run at one wave per SIMD instead of two
    // (62.0 -> 65.5 us at fc2).
    if (tiles > cus && kp.njt <= 4 && kp.K >= 8192) {
      launch_k1_as<FMT, DT, false, 2>(kp, Mp, st);
      return;
    }
  }
  launch_k1_as<FMT, DT, false>(kp, Mp, st);
}

// the down-projection alone (njt > 0)
template <int FMT, int DT>
void launch_k1_proj(const K1Params& kp, int64_t Mp, hipStream_t st) {
  const dim3 grid(unsigned(Mp / 16)), block(256);
  auto red_bytes = [](int njt) { return size_t(4) * size_t(njt) * 64 * 16 + K1_XBUF_BYTES; };
  if (kp.njt <= 2) launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, 2, false, false>), grid, block, red_bytes(2), st, kp);
  else if (kp.njt <= 4) launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, 4, false, false>), grid, block, red_bytes(4), st, kp);
  else launch(SVDQ_KERNEL_ACT, (k1_act<FMT, DT, MAXJT, false, false>), grid, block, red_bytes(MAXJT), st, kp);
}

template <int DT>
void launch_k1_w8(const K1Params& kp, int64_t Mp, hipStream_t st) {
  const dim3 grid(unsigned(Mp / 16)), block(256);
  if (kp.njt == 0) launch(SVDQ_KERNEL_ACT, (k1_w8<DT, 0>), grid, block, 0, st, kp);
  else if (kp.njt == 1) launch(SVDQ_KERNEL_ACT, (k1_w8<DT, 1>), grid, block, 0, st, kp);
  else if (kp.njt <= 2) launch(SVDQ_KERNEL_ACT, (k1_w8<DT, 2>), grid, block, 0, st, kp);
  else if (kp.njt <= 4) launch(SVDQ_KERNEL_ACT, (k1_w8<DT, 4>), grid, block, 0, st, kp);
  else launch(SVDQ_KERNEL_ACT, (k1_w8<DT, MAXJT>), grid, block, 0, st, kp);
}

// (the GEMM launchers return the number of workgroups they launch)
template <int DT>
unsigned launch_k2_int4(const K2Params& kp, int64_t Mp, bool gelu, hipStream_t st) {
  dim3 grid(unsigned(kp.N / 128), unsigned(Mp / 128));
  if (gelu) launch(SVDQ_KERNEL_GEMM, (k2_int4<DT, true>), grid, dim3(256), 0, st, kp);
  else launch(SVDQ_KERNEL_GEMM, (k2_int4<DT, false>), grid, dim3(256), 0, st, kp);
  return grid.x * grid.y;
}

// Tiles per XCD for k2_mx (T tiles, `slots` workgroups resident per XCD).
// Evenly by default; with the staggered start (odd XCDs begin later), the
// odd XCDs take whole rounds one fewer than the even ones need, so their
// late start ends no later than the even XCDs' last round, as long as the
// even XCDs then need no more rounds than an even split would.  Returns the
// workgroups to launch (8 x the largest count).
unsigned set_xcd_split(MxParams& mp, unsigned T, int slots) {
  unsigned cnt[8];
  for (int x = 0; x < 8; ++x) cnt[x] = T / 8 + (unsigned(x) < T % 8 ? 1u : 0u);
  if (slots > 0) {
    const unsigned rounds = (cnt[0] + unsigned(slots) - 1) / unsigned(slots);   // of the even split
    const unsigned odd = (rounds - 1) * unsigned(slots);
    if (rounds >= 2 && T > 4 * odd) {
      const unsigned rest = T - 4 * odd;   // over the four even XCDs
      if ((rest + 3) / 4 <= rounds * unsigned(slots)) {
        for (int x = 0; x < 8; ++x) cnt[x] = (x & 1) ? odd : rest / 4 + (unsigned(x >> 1) < rest % 4 ? 1u : 0u);
      }
    }
  }
  unsigned start = 0, mx = 0;
  for (int x = 0; x < 8; ++x) {
    mp.xcd_start[x] = int(start);
    mp.xcd_count[x] = int(cnt[x]);
    start += cnt[x];
    mx = cnt[x] > mx ? cnt[x] : mx;
  }
  return 8 * mx;
}

MxParams mx_params(const K2Params& kp, const svdq::WsOffsets& w) {
  MxParams mp = {};
  mp.wq = kp.wq; mp.sw = kp.sw; mp.l2 = kp.l2; mp.bias = kp.bias; mp.xq = kp.xq; mp.sx = kp.sx; mp.t = kp.t;
  mp.Y = kp.Y; mp.ldy = kp.ldy; mp.M = kp.M; mp.N = kp.N; mp.K = kp.K; mp.slots = kp.slots;
  mp.nchunks16 = kp.nchunks16;
  mp.tiles_n = int(svdq::ceil_div(kp.N, 256));
  mp.tiles_m = int(w.Mp / 256);
  mp.tiles_m_pad32 = int(w.Mp / 32);
  mp.off_wq = int(kp.wq - reinterpret_cast<const uint8_t*>(kp.l2));
  mp.off_sw = int(kp.sw - reinterpret_cast<const uint8_t*>(kp.l2));
  mp.off_sx = int(kp.sx - kp.xq);
  mp.off_t = int(reinterpret_cast<const uint8_t*>(kp.t) - kp.xq);
  mp.trace = kp.trace;
  set_xcd_split(mp, unsigned(mp.tiles_n) * unsigned(mp.tiles_m), 0);
  return mp;
}

// staggered start (stagger_start) for launches of more than three rounds
constexpr int kStaggerSleeps = 2;
void set_stagger(MxParams& mp, unsigned wgs, int per_cu) {
  const int round = per_cu * device_cus();
  mp.stagger_wgs = int64_t(wgs) > 3 * int64_t(round) ? round : 0;
  mp.stagger_sleeps = kStaggerSleeps;
}

template <int DT, bool I8 = false>
unsigned launch_k2_mx(const K2Params& kp, const svdq::WsOffsets& w, bool gelu, hipStream_t st) {
  MxParams mp = mx_params(kp, w);
  const unsigned T = unsigned(mp.tiles_n) * unsigned(mp.tiles_m);   // 256 x 256 tiles, one per workgroup
  set_stagger(mp, T, 1);
  const unsigned G = mp.stagger_wgs > 0 ? set_xcd_split(mp, T, device_cus() / 8) : T;
  if (gelu) launch(SVDQ_KERNEL_GEMM, (k2_mx<DT, true, false, I8>), dim3(G), dim3(256), 0, st, mp);
  else launch(SVDQ_KERNEL_GEMM, (k2_mx<DT, false, false, I8>), dim3(G), dim3(256), 0, st, mp);
  return G;
}

template <int DT, class C>
unsigned launch_k2_mx8(const K2Params& kp, const svdq::WsOffsets& w, bool gelu, hipStream_t st) {
  MxParams mp = mx_params(kp, w);
  mp.tiles_n = int(svdq::ceil_div(kp.N, C::TN));
  mp.tiles_m = int(svdq::ceil_div(w.Mp, C::TM));
  const unsigned T = unsigned(mp.tiles_n) * unsigned(mp.tiles_m);
  set_stagger(mp, T, C::WG_PER_CU);
  if (gelu) launch(SVDQ_KERNEL_GEMM, (k2_mx8<DT, true, C>), dim3(T), dim3(64 * C::NW), 0, st, mp);
  else launch(SVDQ_KERNEL_GEMM, (k2_mx8<DT, false, C>), dim3(T), dim3(64 * C::NW), 0, st, mp);
  return T;
}

// MXFP4 GEMM.  Without GELU: k2_mx (256 x 256 tiles, four waves, one per
// SIMD).  With GELU: k2_mx8 with 192 x 192 tiles two to a compute unit, so
// one workgroup's GELU epilogue (VALU work after the K loop) runs under the
// other's MFMAs.  Measured on the FLUX fc1 shape, same process, interleaved
// rounds: without GELU the two kernels and an eight-wave 384 x 192 variant
// (three whole rounds) are within 3% of one another -- the clock falls to
// the power limit either way -- while with GELU the paired tiles take 134 us
// against 145 us.
template <int DT>
unsigned launch_k2_mx4(const K2Params& kp, const svdq::WsOffsets& w, bool gelu, hipStream_t st) {
  if (gelu) return launch_k2_mx8<DT, mx8::Pair>(kp, w, true, st);
  return launch_k2_mx<DT>(kp, w, false, st);
}

// chained MXFP4 GEMM: with GELU the paired 192 x 192 tiles (as unchained),
// else k2_mx; returns the partial-slab width (this layer's tile columns)
template <int DT>
int launch_k2_mx8_chain(MxParams mp, int64_t Mp, hipStream_t st) {
  using C = mx8::Pair;
  mp.tiles_n = int(svdq::ceil_div(mp.N, C::TN));
  mp.tiles_m = int(svdq::ceil_div(Mp, C::TM));
  const unsigned T = unsigned(mp.tiles_n) * unsigned(mp.tiles_m);
  set_stagger(mp, T, C::WG_PER_CU);
  launch(SVDQ_KERNEL_GEMM, (k2_mx8<DT, true, C, true>), dim3(T), dim3(64 * C::NW), 0, st, mp);
  return C::TN;
}

template <int DT>
void launch_k2_mx_chain(MxParams mp, bool gelu, hipStream_t st) {
  const unsigned T = unsigned(mp.tiles_n) * unsigned(mp.tiles_m);
  set_stagger(mp, T, 1);
  const unsigned G = mp.stagger_wgs > 0 ? set_xcd_split(mp, T, device_cus() / 8) : T;
  if (gelu) launch(SVDQ_KERNEL_GEMM, (k2_mx<DT, true, true>), dim3(G), dim3(256), 0, st, mp);
  else launch(SVDQ_KERNEL_GEMM, (k2_mx<DT, false, true>), dim3(G), dim3(256), 0, st, mp);
}

template <int DT, int FMT>
void launch_k_up(const UpParams& up, bool gelu, hipStream_t st) {
  const int rows = FMT == SVDQ_FMT_MXFP4_G32 ? 128 : 64;
  const dim3 grid(unsigned(up.N / 128), unsigned(svdq::ceil_div(up.M, rows)));
  if (gelu) launch(SVDQ_KERNEL_OTHER, (k_up<DT, FMT, true>), grid, dim3(256), 0, st, up);
  else launch(SVDQ_KERNEL_OTHER, (k_up<DT, FMT, false>), grid, dim3(256), 0, st, up);
}

svdq_status check_device_layer(const svdq_layer* L) {
  svdq_status s = svdq::validate_layer(L);
  if (s != SVDQ_OK) return s;
  if (!L->blob_on_device) return SVDQ_ERR_INVALID_ARG;
  if (!aligned(L->blob, 256)) return SVDQ_ERR_INVALID_ARG;
  return SVDQ_OK;
}

}  // namespace

// ------------------------------------------------------------- GEMM tracing
// Library-owned trace of the last traced GEMM launch on each device (4
// counters per workgroup, see trace_mark); its device address is looked up
// once per device.
static __device__ unsigned long long trace_buf[kTraceMax * 4];

namespace {

struct TraceState {
  std::mutex mu;
  unsigned long long* ptr[64] = {};
  unsigned n[64] = {};       // workgroups of the last traced launch
};
TraceState g_trace;

svdq_status trace_ptr(unsigned long long** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SVDQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_trace.mu);
  if (g_trace.ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(trace_buf)) != hipSuccess || p == nullptr) return SVDQ_ERR_HIP;
    g_trace.ptr[dev] = static_cast<unsigned long long*>(p);
  }
  *out = g_trace.ptr[dev];
  return SVDQ_OK;
}

void trace_set_count(unsigned n) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return;
  std::lock_guard<std::mutex> lock(g_trace.mu);
  g_trace.n[dev] = n < unsigned(kTraceMax) ? n : unsigned(kTraceMax);
}

enum K1Mode { K1_BOTH, K1_QUANT, K1_PROJ };

// K1 on checked arguments: codes and scales, T, or both
void run_k1(const svdq_layer* L, const void* X_dev, int64_t M, int64_t ldx, uint8_t* ws, const svdq::WsOffsets& w,
            K1Mode mode, hipStream_t stream) {
  const uint8_t* blob = static_cast<const uint8_t*>(L->blob);
  K1Params kp;
  kp.X = static_cast<const uint16_t*>(X_dev);
  kp.ldx = ldx; kp.M = M; kp.K = L->K;
  kp.invlam = reinterpret_cast<const float*>(blob + L->off_invlam);
  kp.l1x = reinterpret_cast<const uint16_t*>(blob + L->off_l1x);
  kp.slots = L->rank_slots;
  // 16-column tiles of T: INT4 fills whole 32-rank chunks (its L1x and T
  // tiling); the MX low-rank layout (MXFP4 and INT8) takes single tiles
  kp.njt = mode == K1_QUANT ? 0
           : L->fmt == SVDQ_FMT_INT4_G64 ? 2 * int(svdq::ceil_div(L->rank_active, 32))
                                         : int(svdq::ceil_div(L->rank_active, 16));
  kp.xq = ws + w.xq; kp.sx = ws + w.sx; kp.t = reinterpret_cast<uint16_t*>(ws + w.t);
  if (L->fmt == SVDQ_FMT_INT8_W8A8) {
    // one kernel for codes, scales and T (the separate-pass modes are not built for INT8)
    if (L->dtype == SVDQ_BF16) launch_k1_w8<SVDQ_BF16>(kp, w.Mp, stream);
    else launch_k1_w8<SVDQ_F16>(kp, w.Mp, stream);
    return;
  }
  if (mode == K1_PROJ) {
    if (kp.njt == 0) return;
    if (L->fmt == SVDQ_FMT_INT4_G64) {
      if (L->dtype == SVDQ_BF16) launch_k1_proj<SVDQ_FMT_INT4_G64, SVDQ_BF16>(kp, w.Mp, stream);
      else launch_k1_proj<SVDQ_FMT_INT4_G64, SVDQ_F16>(kp, w.Mp, stream);
    } else {
      if (L->dtype == SVDQ_BF16) launch_k1_proj<SVDQ_FMT_MXFP4_G32, SVDQ_BF16>(kp, w.Mp, stream);
      else launch_k1_proj<SVDQ_FMT_MXFP4_G32, SVDQ_F16>(kp, w.Mp, stream);
    }
    return;
  }
  if (L->fmt == SVDQ_FMT_INT4_G64) {
    if (L->dtype == SVDQ_BF16) launch_k1<SVDQ_FMT_INT4_G64, SVDQ_BF16>(kp, w.Mp, stream);
    else launch_k1<SVDQ_FMT_INT4_G64, SVDQ_F16>(kp, w.Mp, stream);
  } else {
    if (L->dtype == SVDQ_BF16) launch_k1<SVDQ_FMT_MXFP4_G32, SVDQ_BF16>(kp, w.Mp, stream);
    else launch_k1<SVDQ_FMT_MXFP4_G32, SVDQ_F16>(kp, w.Mp, stream);
  }
}

K2Params k2_params(const svdq_layer* L, int64_t M, void* Y_dev, int64_t ldy, const uint8_t* ws,
                   const svdq::WsOffsets& w, bool lowrank) {
  const uint8_t* blob = static_cast<const uint8_t*>(L->blob);
  K2Params kp;
  kp.wq = blob + L->off_wq;
  kp.sw = blob + L->off_sw;
  kp.l2 = reinterpret_cast<const uint16_t*>(blob + L->off_l2);
  kp.bias = reinterpret_cast<const float*>(blob + L->off_bias);
  kp.xq = ws + w.xq; kp.sx = ws + w.sx;
  kp.t = reinterpret_cast<const uint16_t*>(ws + w.t);
  kp.Y = static_cast<uint16_t*>(Y_dev);
  kp.ldy = ldy; kp.M = M; kp.N = L->N; kp.K = L->K;
  kp.slots = L->rank_slots;
  const int ra = lowrank ? L->rank_active : 0;
  kp.nchunks = int(svdq::ceil_div(ra, 32));
  kp.nchunks16 = int(svdq::ceil_div(ra, 16));
  kp.trace = nullptr;
  kp.nx_invlam = nullptr; kp.nx_l1x = nullptr; kp.nx_xq = nullptr; kp.nx_sx = nullptr; kp.nx_tp = nullptr;
  kp.nx_Mp = 0; kp.nx_slots = 0; kp.nx_njt = 0;
  return kp;
}

// K2 on checked arguments; lowrank = false leaves the low-rank branch out;
// trace: device trace records or null
void run_k2(const svdq_layer* L, int64_t M, void* Y_dev, int64_t ldy, const uint8_t* ws, const svdq::WsOffsets& w,
            bool gelu, bool lowrank, hipStream_t stream, unsigned long long* trace = nullptr) {
  K2Params kp = k2_params(L, M, Y_dev, ldy, ws, w, lowrank);
  kp.trace = trace;
  unsigned nwg = 0;
  if (L->fmt == SVDQ_FMT_INT8_W8A8) {
    if (L->dtype == SVDQ_BF16) nwg = launch_k2_mx<SVDQ_BF16, true>(kp, w, gelu, stream);
    else nwg = launch_k2_mx<SVDQ_F16, true>(kp, w, gelu, stream);
  } else if (L->fmt == SVDQ_FMT_INT4_G64) {
    if (L->dtype == SVDQ_BF16) nwg = launch_k2_int4<SVDQ_BF16>(kp, w.Mp, gelu, stream);
    else nwg = launch_k2_int4<SVDQ_F16>(kp, w.Mp, gelu, stream);
  } else {
    if (L->dtype == SVDQ_BF16) nwg = launch_k2_mx4<SVDQ_BF16>(kp, w, gelu, stream);
    else nwg = launch_k2_mx4<SVDQ_F16>(kp, w, gelu, stream);
  }
  if (trace != nullptr) trace_set_count(nwg);
}

// the MXFP4 GEMM addresses the blob from L2 and the workspace from the
// activation codes with 31-bit offsets
bool mx_offsets_fit(const svdq_layer* L, const svdq::WsOffsets& w) {
  const size_t lim = size_t(1) << 31;
  if (L->fmt == SVDQ_FMT_INT4_G64) {
    // the INT4 GEMM's buffer loads: codes and scales of each operand
    return size_t(L->N) * size_t(L->K) / 2 < lim && size_t(w.Mp) * size_t(L->K) / 2 < lim;
  }
  return L->off_bias + size_t(L->N) * 4 - L->off_l2 < lim && w.total - w.xq < lim;
}

// the unfused baseline's up-projection pass: Y = round16(GELU?(Y + T L2))
void run_up(const svdq_layer* L, int64_t M, void* Y_dev, int64_t ldy, const uint8_t* ws, const svdq::WsOffsets& w,
            bool gelu, hipStream_t stream) {
  const uint8_t* blob = static_cast<const uint8_t*>(L->blob);
  UpParams up;
  up.l2 = reinterpret_cast<const uint16_t*>(blob + L->off_l2);
  up.t = reinterpret_cast<const uint16_t*>(ws + w.t);
  up.Y = static_cast<uint16_t*>(Y_dev);
  up.ldy = ldy; up.M = M; up.N = L->N;
  up.slots = L->rank_slots;
  const bool mx = L->fmt == SVDQ_FMT_MXFP4_G32;
  up.nchunks = int(svdq::ceil_div(L->rank_active, mx ? 16 : 32));
  if (mx) {
    if (L->dtype == SVDQ_BF16) launch_k_up<SVDQ_BF16, SVDQ_FMT_MXFP4_G32>(up, gelu, stream);
    else launch_k_up<SVDQ_F16, SVDQ_FMT_MXFP4_G32>(up, gelu, stream);
  } else {
    if (L->dtype == SVDQ_BF16) launch_k_up<SVDQ_BF16, SVDQ_FMT_INT4_G64>(up, gelu, stream);
    else launch_k_up<SVDQ_F16, SVDQ_FMT_INT4_G64>(up, gelu, stream);
  }
}

constexpr unsigned SVDQ_FLAGS_ALL =
    unsigned(SVDQ_FLAG_GELU) | unsigned(SVDQ_FLAG_UNFUSED_LOWRANK) | unsigned(SVDQ_FLAG_TRACE);

svdq_status check_x(const svdq_layer* L, const void* X_dev, int64_t ldx) {
  if (!X_dev) return SVDQ_ERR_INVALID_ARG;
  if (ldx < L->K || ldx % 8 != 0 || !aligned(X_dev, 16)) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}
svdq_status check_y(const svdq_layer* L, const void* Y_dev, int64_t ldy) {
  if (!Y_dev) return SVDQ_ERR_INVALID_ARG;
  if (ldy < L->N || ldy % 8 != 0 || !aligned(Y_dev, 16)) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}
svdq_status check_ws(const svdq_layer* L, int64_t M, const void* ws_dev, size_t ws_bytes, svdq::WsOffsets* w) {
  if (!ws_dev) return SVDQ_ERR_INVALID_ARG;
  *w = svdq::ws_offsets(M, L->K, L->rank_slots, L->fmt);
  if (ws_bytes < w->total) return SVDQ_ERR_CAPACITY;
  if (!aligned(ws_dev, 256)) return SVDQ_ERR_INVALID_ARG;
  return SVDQ_OK;
}

// Epilogue chaining: `first` feeds `next` (same dtype, MXFP4 both,
// first->N == next->K).  The fp32 partial down-projections of `next` sit
// after `first`'s own workspace.
svdq_status check_chain(const svdq_layer* A, const svdq_layer* B) {
  svdq_status st = check_device_layer(A);
  if (st != SVDQ_OK || (st = check_device_layer(B)) != SVDQ_OK) return st;
  if (A->dtype != B->dtype) return SVDQ_ERR_INVALID_ARG;
  if (A->N != B->K) return SVDQ_ERR_SHAPE;
  // pairs of one 4-bit format: MXFP4 -> MXFP4 or INT4 -> INT4
  const bool mx = A->fmt == SVDQ_FMT_MXFP4_G32 && B->fmt == SVDQ_FMT_MXFP4_G32;
  const bool i4 = A->fmt == SVDQ_FMT_INT4_G64 && B->fmt == SVDQ_FMT_INT4_G64;
  if (!mx && !i4) return SVDQ_ERR_UNSUPPORTED;
  return SVDQ_OK;
}
size_t chain_partials_offset(const svdq::WsOffsets& w) { return svdq::align256(w.total); }
// output columns of `first` per partial slab: the GEMM's workgroup tile
// width (the workspace holds slabs for the narrowest, 192-column tiles of
// the paired MXFP4 GEMM)
int64_t chain_slab_cols(const svdq_layer* A) { return A->fmt == SVDQ_FMT_INT4_G64 ? 128 : 192; }
size_t chain_partials_bytes(const svdq_layer* A, const svdq_layer* B, const svdq::WsOffsets& w) {
  return size_t(svdq::ceil_div(A->N, chain_slab_cols(A))) * size_t(w.Mp) * size_t(B->rank_slots) * 4;
}

}  // namespace

extern "C" svdq_status svdq_chain_workspace_size(const svdq_layer* first, const svdq_layer* next, int64_t M,
                                                 size_t* bytes) {
  svdq_status st = check_chain(first, next);
  if (st != SVDQ_OK) return st;
  if (M < 0 || !bytes) return SVDQ_ERR_INVALID_ARG;
  const svdq::WsOffsets w = svdq::ws_offsets(M, first->K, first->rank_slots, first->fmt);
  *bytes = chain_partials_offset(w) + chain_partials_bytes(first, next, w);
  return SVDQ_OK;
}

extern "C" svdq_status svdq_linear_forward_chain(const svdq_layer* first, const svdq_layer* next, const void* X_dev,
                                                 int64_t M, int64_t ldx, void* Y_dev, int64_t ldy, void* ws_dev,
                                                 size_t ws_bytes, void* ws_next_dev, size_t ws_next_bytes,
                                                 unsigned flags, hipStream_t stream) {
  svdq_status st = check_chain(first, next);
  if (st != SVDQ_OK) return st;
  if (M < 0 || (flags & ~unsigned(SVDQ_FLAG_GELU)) != 0u) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  svdq::WsOffsets w, wn;
  if ((st = check_x(first, X_dev, ldx)) != SVDQ_OK || (st = check_ws(next, M, ws_next_dev, ws_next_bytes, &wn)) != SVDQ_OK)
    return st;
  if (Y_dev && (st = check_y(first, Y_dev, ldy)) != SVDQ_OK) return st;
  if (!ws_dev) return SVDQ_ERR_INVALID_ARG;
  w = svdq::ws_offsets(M, first->K, first->rank_slots, first->fmt);
  if (ws_bytes < chain_partials_offset(w) + chain_partials_bytes(first, next, w)) return SVDQ_ERR_CAPACITY;
  if (!aligned(ws_dev, 256)) return SVDQ_ERR_INVALID_ARG;
  if (!mx_offsets_fit(first, w)) return SVDQ_ERR_UNSUPPORTED;
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  uint8_t* wsn = static_cast<uint8_t*>(ws_next_dev);
  const uint8_t* nblob = static_cast<const uint8_t*>(next->blob);
  const bool gelu = (flags & SVDQ_FLAG_GELU) != 0u;
  const bool i4 = first->fmt == SVDQ_FMT_INT4_G64;
  run_k1(first, X_dev, M, ldx, ws, w, K1_BOTH, stream);
  K2Params kp = k2_params(first, M, Y_dev, ldy, ws, w, true);
  kp.nx_invlam = reinterpret_cast<const float*>(nblob + next->off_invlam);
  kp.nx_l1x = reinterpret_cast<const uint16_t*>(nblob + next->off_l1x);
  kp.nx_xq = wsn + wn.xq;
  kp.nx_sx = wsn + wn.sx;
  kp.nx_tp = reinterpret_cast<float*>(ws + chain_partials_offset(w));
  kp.nx_Mp = w.Mp;
  kp.nx_slots = next->rank_slots;
  // T column tiles of 16: INT4 fills whole 32-rank chunks (its T layout)
  kp.nx_njt = i4 ? 2 * int(svdq::ceil_div(next->rank_active, 32)) : int(svdq::ceil_div(next->rank_active, 16));
  int64_t slab_cols = 128;
  if (i4) {
    const dim3 grid(unsigned(kp.N / 128), unsigned(w.Mp / 128));
    if (first->dtype == SVDQ_BF16) {
      if (gelu) launch(SVDQ_KERNEL_GEMM, (k2_int4<SVDQ_BF16, true, true>), grid, dim3(256), 0, stream, kp);
      else launch(SVDQ_KERNEL_GEMM, (k2_int4<SVDQ_BF16, false, true>), grid, dim3(256), 0, stream, kp);
    } else {
      if (gelu) launch(SVDQ_KERNEL_GEMM, (k2_int4<SVDQ_F16, true, true>), grid, dim3(256), 0, stream, kp);
      else launch(SVDQ_KERNEL_GEMM, (k2_int4<SVDQ_F16, false, true>), grid, dim3(256), 0, stream, kp);
    }
  } else {
    MxParams mp = mx_params(kp, w);
    mp.nx_invlam = kp.nx_invlam;
    mp.nx_l1x = kp.nx_l1x;
    mp.nx_xq = kp.nx_xq;
    mp.nx_sx = kp.nx_sx;
    mp.nx_tp = kp.nx_tp;
    mp.nx_Mp = kp.nx_Mp;
    mp.nx_slots = kp.nx_slots;
    mp.nx_njt = kp.nx_njt;
    if (gelu) {
      slab_cols = first->dtype == SVDQ_BF16 ? launch_k2_mx8_chain<SVDQ_BF16>(mp, w.Mp, stream)
                                            : launch_k2_mx8_chain<SVDQ_F16>(mp, w.Mp, stream);
    } else {
      if (first->dtype == SVDQ_BF16) launch_k2_mx_chain<SVDQ_BF16>(mp, false, stream);
      else launch_k2_mx_chain<SVDQ_F16>(mp, false, stream);
      slab_cols = 256;
    }
  }
  if (kp.nx_njt > 0) {
    TfinParams tf;
    tf.tp = kp.nx_tp;
    tf.t = reinterpret_cast<uint16_t*>(wsn + wn.t);
    tf.Mp = w.Mp;
    tf.slots = next->rank_slots;
    tf.nparts = int(svdq::ceil_div(first->N, slab_cols));
    tf.ncols4 = 4 * kp.nx_njt;
    const int64_t n = w.Mp * tf.ncols4;
    const dim3 grid(unsigned((n + 63) / 64));
    if (i4) {
      if (first->dtype == SVDQ_BF16) launch(SVDQ_KERNEL_OTHER, (k_tfin<SVDQ_BF16, SVDQ_FMT_INT4_G64>), grid, dim3(256), 0, stream, tf);
      else launch(SVDQ_KERNEL_OTHER, (k_tfin<SVDQ_F16, SVDQ_FMT_INT4_G64>), grid, dim3(256), 0, stream, tf);
    } else {
      if (first->dtype == SVDQ_BF16) launch(SVDQ_KERNEL_OTHER, (k_tfin<SVDQ_BF16, SVDQ_FMT_MXFP4_G32>), grid, dim3(256), 0, stream, tf);
      else launch(SVDQ_KERNEL_OTHER, (k_tfin<SVDQ_F16, SVDQ_FMT_MXFP4_G32>), grid, dim3(256), 0, stream, tf);
    }
  }
  return launch_ok();
}

extern "C" svdq_status svdq_quantize_activations(const svdq_layer* L, const void* X_dev, int64_t M, int64_t ldx,
                                                 void* ws_dev, size_t ws_bytes, hipStream_t stream) {
  svdq_status st = check_device_layer(L);
  if (st != SVDQ_OK) return st;
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  svdq::WsOffsets w;
  if ((st = check_x(L, X_dev, ldx)) != SVDQ_OK || (st = check_ws(L, M, ws_dev, ws_bytes, &w)) != SVDQ_OK) return st;
  run_k1(L, X_dev, M, ldx, static_cast<uint8_t*>(ws_dev), w, K1_BOTH, stream);
  return launch_ok();
}

extern "C" svdq_status svdq_gemm_forward(const svdq_layer* L, int64_t M, void* Y_dev, int64_t ldy,
                                         const void* ws_dev, size_t ws_bytes, unsigned flags, hipStream_t stream) {
  svdq_status st = check_device_layer(L);
  if (st != SVDQ_OK) return st;
  if (M < 0 || (flags & ~unsigned(SVDQ_FLAG_GELU | SVDQ_FLAG_TRACE)) != 0u) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  svdq::WsOffsets w;
  if ((st = check_y(L, Y_dev, ldy)) != SVDQ_OK || (st = check_ws(L, M, ws_dev, ws_bytes, &w)) != SVDQ_OK) return st;
  if (!mx_offsets_fit(L, w)) return SVDQ_ERR_UNSUPPORTED;
  unsigned long long* trace = nullptr;
  if ((flags & SVDQ_FLAG_TRACE) != 0u && (st = trace_ptr(&trace)) != SVDQ_OK) return st;
  run_k2(L, M, Y_dev, ldy, static_cast<const uint8_t*>(ws_dev), w, (flags & SVDQ_FLAG_GELU) != 0u, true, stream, trace);
  return launch_ok();
}

extern "C" svdq_status svdq_linear_forward(const svdq_layer* L, const void* X_dev, int64_t M, int64_t ldx,
                                           void* Y_dev, int64_t ldy, void* ws_dev, size_t ws_bytes, unsigned flags,
                                           hipStream_t stream) {
  svdq_status st = check_device_layer(L);
  if (st != SVDQ_OK) return st;
  if (M < 0 || (flags & ~SVDQ_FLAGS_ALL) != 0u) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  svdq::WsOffsets w;
  if ((st = check_x(L, X_dev, ldx)) != SVDQ_OK || (st = check_y(L, Y_dev, ldy)) != SVDQ_OK ||
      (st = check_ws(L, M, ws_dev, ws_bytes, &w)) != SVDQ_OK)
    return st;
  if (!mx_offsets_fit(L, w)) return SVDQ_ERR_UNSUPPORTED;
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  const bool gelu = (flags & SVDQ_FLAG_GELU) != 0u;
  if ((flags & SVDQ_FLAG_UNFUSED_LOWRANK) != 0u && L->fmt == SVDQ_FMT_INT8_W8A8) return SVDQ_ERR_UNSUPPORTED;
  unsigned long long* trace = nullptr;
  if ((flags & SVDQ_FLAG_TRACE) != 0u && (st = trace_ptr(&trace)) != SVDQ_OK) return st;
  if ((flags & SVDQ_FLAG_UNFUSED_LOWRANK) == 0u || L->rank_active == 0) {
    run_k1(L, X_dev, M, ldx, ws, w, K1_BOTH, stream);
    run_k2(L, M, Y_dev, ldy, ws, w, gelu, true, stream, trace);
  } else {
    // the low-rank branch as separate passes: quantize, down-project (a
    // second read of X), 4-bit GEMM + bias, then Y += T L2 (+ GELU)
    run_k1(L, X_dev, M, ldx, ws, w, K1_QUANT, stream);
    run_k1(L, X_dev, M, ldx, ws, w, K1_PROJ, stream);
    run_k2(L, M, Y_dev, ldy, ws, w, false, false, stream, trace);
    run_up(L, M, Y_dev, ldy, ws, w, gelu, stream);
  }
  return launch_ok();
}

// ------------------------------------------------- forward without allocation
// Library-owned workspace for svdq_linear_forward_noalloc: one copy per GPU
// (each device that loads this code object holds its own), kept until the
// process ends.  Host code never passes the symbol itself to a kernel: its
// device address comes from hipGetSymbolAddress, looked up once per device.
static __device__ __attribute__((aligned(256))) uint8_t scratch[SVDQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of this device's scratch array (looked up on first use)
svdq_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SVDQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SVDQ_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SVDQ_OK;
}
}  // namespace

extern "C" svdq_status svdq_linear_forward_noalloc(const svdq_layer* L, const void* X_dev, int64_t M, int64_t ldx,
                                                   void* Y_dev, int64_t ldy, unsigned flags, hipStream_t stream) {
  svdq_status st = check_device_layer(L);
  if (st != SVDQ_OK) return st;
  if (M < 0 || (flags & ~SVDQ_FLAGS_ALL) != 0u) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  // the workspace this forward needs must fit the library's array
  const svdq::WsOffsets w = svdq::ws_offsets(M, L->K, L->rank_slots, L->fmt);
  if (w.total > size_t(SVDQ_NOALLOC_SCRATCH_BYTES)) return SVDQ_ERR_CAPACITY;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != SVDQ_OK) return st;
  return svdq_linear_forward(L, X_dev, M, ldx, Y_dev, ldy, ws, size_t(SVDQ_NOALLOC_SCRATCH_BYTES), flags, stream);
}

extern "C" svdq_status svdq_trace_read(unsigned long long* records, int max_records, int* n_records,
                                       double* wall_hz) {
  if (!n_records || !wall_hz || max_records < 0 || (max_records > 0 && !records)) return SVDQ_ERR_INVALID_ARG;
  int dev = -1, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SVDQ_ERR_HIP;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return SVDQ_ERR_HIP;
  unsigned long long* ptr = nullptr;
  svdq_status st = trace_ptr(&ptr);
  if (st != SVDQ_OK) return st;
  unsigned n = 0;
  {
    std::lock_guard<std::mutex> lock(g_trace.mu);
    n = g_trace.n[dev];
  }
  *n_records = int(n);
  *wall_hz = double(khz) * 1e3;
  const unsigned k = n < unsigned(max_records) ? n : unsigned(max_records);
  if (k == 0) return SVDQ_OK;
  if (hipDeviceSynchronize() != hipSuccess) return SVDQ_ERR_HIP;
  if (hipMemcpy(records, ptr, size_t(k) * 4 * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
    return SVDQ_ERR_HIP;
  return SVDQ_OK;
}

namespace {
void timing_release(KernelTiming& t) {
  for (hipEvent_t e : t.ev)
    if (e) (void)hipEventDestroy(e);
  t.ev.clear();
  t.kind.clear();
  t.used = 0;
  t.on = false;
}
}  // namespace

extern "C" svdq_status svdq_timing_start(int capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return SVDQ_ERR_INVALID_ARG;
  KernelTiming& t = t_timing;
  timing_release(t);
  t.ev.assign(size_t(2) * size_t(capacity), nullptr);
  t.kind.assign(size_t(capacity), 0);
  for (hipEvent_t& e : t.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      timing_release(t);
      return SVDQ_ERR_HIP;
    }
  }
  t.on = true;
  return SVDQ_OK;
}

extern "C" svdq_status svdq_timing_stop(int* kinds, float* ms, int max_launches, int* n_launches) {
  if (!n_launches || max_launches < 0 || (max_launches > 0 && (!kinds || !ms))) return SVDQ_ERR_INVALID_ARG;
  KernelTiming& t = t_timing;
  t.on = false;
  const size_t n = t.used;
  *n_launches = int(n);
  svdq_status st = SVDQ_OK;
  for (size_t i = 0; i < n && i < size_t(max_launches); ++i) {
    float v = 0.0f;
    if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&v, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) {
      st = SVDQ_ERR_HIP;
      break;
    }
    kinds[i] = t.kind[i];
    ms[i] = v;
  }
  timing_release(t);
  return st;
}

extern "C" svdq_status svdq_activation_absmax(const void* X_dev, int64_t M, int64_t K, int64_t ldx,
                                              svdq_dtype dtype, float* absmax_dev, hipStream_t stream) {
  if (M < 0 || K <= 0 || ldx < K) return SVDQ_ERR_INVALID_ARG;
  if (dtype != SVDQ_F16 && dtype != SVDQ_BF16) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  if (!X_dev || !absmax_dev) return SVDQ_ERR_INVALID_ARG;
  const int64_t rpb = 64;
  dim3 grid(unsigned((K + 255) / 256), unsigned((M + rpb - 1) / rpb));
  const uint16_t* X = static_cast<const uint16_t*>(X_dev);
  if (dtype == SVDQ_BF16) hipLaunchKernelGGL((k_absmax<SVDQ_BF16>), grid, dim3(256), 0, stream, X, M, K, ldx, rpb, absmax_dev);
  else hipLaunchKernelGGL((k_absmax<SVDQ_F16>), grid, dim3(256), 0, stream, X, M, K, ldx, rpb, absmax_dev);
  return launch_ok();
}

extern "C" svdq_status svdq_int4_group_partials(const svdq_layer* L, const void* ws_dev, size_t ws_bytes, int64_t M,
                                                int64_t m0, int64_t nm, int64_t n0, int64_t nn, int64_t g0,
                                                int64_t ng, int32_t* out_dev, hipStream_t stream) {
  svdq_status st = check_device_layer(L);
  if (st != SVDQ_OK) return st;
  if (L->fmt != SVDQ_FMT_INT4_G64) return SVDQ_ERR_UNSUPPORTED;
  if (!ws_dev || !out_dev || M <= 0) return SVDQ_ERR_INVALID_ARG;
  svdq::WsOffsets w = svdq::ws_offsets(M, L->K, L->rank_slots, L->fmt);
  if (ws_bytes < w.total) return SVDQ_ERR_CAPACITY;
  if (m0 < 0 || n0 < 0 || g0 < 0 || nm <= 0 || nn <= 0 || ng <= 0) return SVDQ_ERR_INVALID_ARG;
  if (m0 % 16 || n0 % 16 || nm % 16 || nn % 16) return SVDQ_ERR_SHAPE;
  if (m0 + nm > w.Mp || n0 + nn > L->N || g0 + ng > L->K / 64) return SVDQ_ERR_SHAPE;
  PartialParams pp;
  pp.wq = static_cast<const uint8_t*>(L->blob) + L->off_wq;
  pp.xq = static_cast<const uint8_t*>(ws_dev) + w.xq;
  pp.out = out_dev;
  pp.K = L->K; pp.m0 = m0; pp.nm = nm; pp.n0 = n0; pp.nn = nn; pp.g0 = g0;
  hipLaunchKernelGGL(k_int4_partials, dim3(unsigned(nn / 16), unsigned(nm / 16), unsigned(ng)), dim3(64), 0, stream, pp);
  return launch_ok();
}
