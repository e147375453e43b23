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

#include <cstdint>

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

template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == SVDQ_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// E2M1 magnitude index of a >= 0: nearest value, ties to the even mantissa, saturating at 6.
__device__ __forceinline__ unsigned e2m1_index(float a) {
  return unsigned(a > 0.25f) + unsigned(a >= 0.75f) + unsigned(a > 1.25f) + unsigned(a >= 1.75f) +
         unsigned(a > 2.5f) + unsigned(a >= 3.5f) + unsigned(a > 5.0f);
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

// One workgroup = 16 tokens; its 4 waves take the 128-deep K steps round robin.
// Lane l holds token (l % 16) and k in [32q, 32q+32) of a step (q = l / 16).
template <int FMT, int DT>
__global__ __launch_bounds__(256) void k1_act(K1Params p) {
  const int mt = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  const int64_t row = int64_t(mt) * 16 + m;
  const bool valid = row < p.M;
  const int nsteps = int(p.K / KSTEP);
  const uint16_t* xrow = p.X + (valid ? row : 0) * p.ldx;

  f32x4 tacc[MAXJT];
#pragma unroll
  for (int j = 0; j < MAXJT; ++j) tacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s = wave; s < nsteps; s += 4) {
    const int k0 = s * KSTEP + q * 32;
    u32x4 xr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xr[i] = valid ? *reinterpret_cast<const u32x4*>(xrow + k0 + 8 * i) : u32x4{0u, 0u, 0u, 0u};
    }
    float xh[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 il = *reinterpret_cast<const f32x4*>(p.invlam + k0 + 4 * i);
      const unsigned w0 = xr[i >> 1][(i & 1) * 2], w1 = xr[i >> 1][(i & 1) * 2 + 1];
      xh[4 * i + 0] = h2f<DT>(w0 & 0xFFFFu) * il[0];
      xh[4 * i + 1] = h2f<DT>(w0 >> 16) * il[1];
      xh[4 * i + 2] = h2f<DT>(w1 & 0xFFFFu) * il[2];
      xh[4 * i + 3] = h2f<DT>(w1 >> 16) * il[3];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(xh[i]));

    uint8_t* frag = p.xq + (size_t(mt) * nsteps + s) * svdq::FRAG_BYTES;
    if constexpr (FMT == SVDQ_FMT_INT4_G64) {
      amax = fmaxf(amax, __shfl_xor(amax, 16));            // the 64-group spans lanes q and q^1
      float sc = fminf(amax / 7.0f, 65504.0f);
      const unsigned sh = f2h<SVDQ_F16>(sc);
      const float s32 = h2f<SVDQ_F16>(sh);
      unsigned d[4] = {0u, 0u, 0u, 0u};
      if (s32 != 0.0f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          float r = rintf(xh[i] / s32);
          r = fminf(fmaxf(r, -7.0f), 7.0f);
          const unsigned c = unsigned(int(r)) & 0xFu;
          d[i >> 3] |= c << (4 * (i & 7));
        }
      }
      // k in [32q, 32q+16) -> slot (m, 2(q%2)), k in [32q+16, 32q+32) -> slot (m, 2(q%2)+1);
      // byte half = 64-group within the step (q / 2)
      const int qa = 2 * (q & 1), half = 8 * (q >> 1);
      *reinterpret_cast<u32x2*>(frag + (m + 16 * qa) * 16 + half) = u32x2{d[0], d[1]};
      *reinterpret_cast<u32x2*>(frag + (m + 16 * (qa + 1)) * 16 + half) = u32x2{d[2], d[3]};
      if ((q & 1) == 0) {
        uint16_t* sxp = reinterpret_cast<uint16_t*>(p.sx);
        sxp[((size_t(mt) * nsteps + s) * 16 + m) * 2 + (q >> 1)] = (uint16_t)sh;
      }
    } else {
      const float tq = amax / 6.0f;
      const unsigned tb = __float_as_uint(tq);
      int e = int((tb >> 23) & 0xFFu) + ((tb & 0x7FFFFFu) != 0u ? 1 : 0);
      if (tq == 0.0f) e = 0;
      e = e > 254 ? 254 : e;
      unsigned d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float u = ldexpf(xh[i], 127 - e);
        const unsigned c = e2m1_index(fabsf(u)) | ((__float_as_uint(xh[i]) >> 28) & 8u);
        d[i >> 3] |= c << (4 * (i & 7));
      }
      *reinterpret_cast<u32x4*>(frag + lane * 16) = u32x4{d[0], d[1], d[2], d[3]};
      // byte (mt % 4) of the dword of tile group mt / 4 (selected by op_sel in the GEMM)
      p.sx[((size_t(mt >> 2) * nsteps + s) * 64 + lane) * 4 + (mt & 3)] = (uint8_t)e;
    }

    // down-projection T^T += L1x^T X^T on the raw 16-bit inputs
    const u32x4* l1 = reinterpret_cast<const u32x4*>(p.l1x) + (size_t(s) * (p.slots / 16)) * 4 * 64;
#pragma unroll
    for (int jt = 0; jt < MAXJT; ++jt) {
      if (jt < p.njt) {
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
          const u32x4 a = l1[(jt * 4 + jp) * 64 + lane];
          tacc[jt] = mfma16<DT>(a, xr[jp], tacc[jt]);
        }
      }
    }
  }

  if (p.njt == 0) return;
  __shared__ f32x4 red[4][MAXJT][64];
#pragma unroll
  for (int jt = 0; jt < MAXJT; ++jt)
    if (jt < p.njt) red[wave][jt][lane] = tacc[jt];
  __syncthreads();
  for (int jt = wave; jt < p.njt; jt += 4) {
    f32x4 v = red[0][jt][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[w][jt][lane];
    // lane holds T[m][16 jt + 4q + i]; place it in the epilogue's B-fragment order
    const int c = jt >> 1;
    const int ldst = m + 16 * (2 * (jt & 1) + (q >> 1));
    const int e0 = 4 * (q & 1);
    const unsigned lo = f2h<DT>(v[0]) | (f2h<DT>(v[1]) << 16);
    const unsigned hi = f2h<DT>(v[2]) | (f2h<DT>(v[3]) << 16);
    uint16_t* dst = p.t + ((size_t(mt) * (p.slots / 32) + c) * 64 + ldst) * 8 + e0;
    *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
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
  int slots, nchunks;
};

__device__ __forceinline__ i32x4 widen_nibbles(unsigned d0, unsigned d1) {
  // 16 signed nibbles -> 16 int8 holding 16*q (even elements first, then odd;
  // both operands use the same order, so the dot product is unchanged)
  return i32x4{int((d0 << 4) & 0xF0F0F0F0u), int((d1 << 4) & 0xF0F0F0F0u), int(d0 & 0xF0F0F0F0u),
               int(d1 & 0xF0F0F0F0u)};
}

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// INT4 GEMM.  One workgroup = 128 output columns x 128 tokens; 4 waves in a
// 2 x 2 grid, each 64 x 64 (4 x 4 MFMA tiles of 16 x 16).
template <int DT, bool GELU>
__global__ __launch_bounds__(256) void k2_int4(K2Params p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t n0 = int64_t(blockIdx.x) * 128 + wn * 64;
  const int64_t m0 = int64_t(blockIdx.y) * 128 + wm * 64;
  const int64_t nt0 = n0 / 16, mt0 = m0 / 16;
  const int nsteps = int(p.K / KSTEP);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4* wq = reinterpret_cast<const u32x4*>(p.wq);
  const u32x4* xq = reinterpret_cast<const u32x4*>(p.xq);

  for (int s = 0; s < nsteps; ++s) {
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = wq[((nt0 + i) * nsteps + s) * 64 + lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = xq[((mt0 + j) * nsteps + s) * 64 + lane];
    {
      // scales: weight side 4 consecutive n x 2 groups per lane, token side 2 groups per lane
      const uint16_t* sw16 = reinterpret_cast<const uint16_t*>(p.sw);
      const uint16_t* sx16 = reinterpret_cast<const uint16_t*>(p.sx);
      float swf[4][2][4], sxf[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sw16 + ((((nt0 + i) * nsteps + s) * 4 + q) * 2) * 4);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) swf[i][g][r] = h2f<SVDQ_F16>((v[g * 2 + (r >> 1)] >> (16 * (r & 1))) & 0xFFFFu);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned v = *reinterpret_cast<const unsigned*>(sx16 + (((mt0 + j) * nsteps + s) * 16 + (lane & 15)) * 2);
        sxf[j][0] = h2f<SVDQ_F16>(v & 0xFFFFu) * (1.0f / 256.0f);
        sxf[j][1] = h2f<SVDQ_F16>(v >> 16) * (1.0f / 256.0f);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        i32x4 ua[4], ub[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ua[i] = widen_nibbles(a[i][2 * g], a[i][2 * g + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) ub[j] = widen_nibbles(b[j][2 * g], b[j][2 * g + 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const i32x4 P = __builtin_amdgcn_mfma_i32_16x16x64_i8(ua[i], ub[j], i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i][j][r] = fmaf(float(P[r]), swf[i][g][r] * sxf[j][g], acc[i][j][r]);
          }
      }
    }
  }

  // epilogue: + T L2 (16-bit MFMA into the same accumulators), + bias, GELU, round, store
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
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<DT>(la[i], tb[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + 16 * i + 4 * q;
    const f32x4 bv = *reinterpret_cast<const f32x4*>(p.bias + n);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + 16 * j + (lane & 15);
      if (m < p.M) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][j][r] + bv[r];
          if constexpr (GELU) v[r] = gelu_erf(v[r]);
        }
        const unsigned lo = f2h<DT>(v[0]) | (f2h<DT>(v[1]) << 16);
        const unsigned hi = f2h<DT>(v[2]) | (f2h<DT>(v[3]) << 16);
        *reinterpret_cast<u32x2*>(p.Y + m * p.ldy + n) = u32x2{lo, hi};
      }
    }
  }
}


// ------------------------------------------------------------ k2_mx (MXFP4)
// One workgroup = 256 output columns x 256 tokens, 4 waves in a 2 x 2 grid,
// each 128 x 128 (8 x 8 tiles of 16 x 16, 256 fp32 accumulators per lane).
// Per 128-deep K step the workgroup stages 16 weight fragments, 16
// activation fragments and their e8m0 scale dwords (34 KB) in LDS with
// direct global->LDS loads; MX_STAGES steps are in flight.  Each wave issues
// 10 of the 40 loads of a step.  The tile order is XCD-aware: consecutive
// tiles of the grouped order land on the same XCD (and its L2).
namespace mx {
constexpr int STAGES = 4;
constexpr int A_OFF = 0;                 // 16 weight fragments
constexpr int B_OFF = 16 * 1024;         // 16 activation fragments
constexpr int SA_OFF = 32 * 1024;        // 4 weight scale dwords x 64 lanes
constexpr int SB_OFF = 32 * 1024 + 1024; // 4 activation scale dwords x 64 lanes
constexpr int STAGE_BYTES = 34 * 1024;
constexpr int GROUP_M = 8;               // m-tiles per group of the tile order
}  // namespace mx

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
  int slots, nchunks;
  int tiles_n, tiles_m;
};


// Scaled FP4 MFMA with the scale bytes picked by op_sel; oa / ob are
// compile-time constants at every call site (unrolled loops), so the switch folds.
__device__ __forceinline__ f32x4 mfma_mx(const i32x8& a, const i32x8& b, f32x4 c, int sa, int sb, int oa, int ob) {
#define SVDQ_MX_CASE(OA, OB) \
  case OA * 4 + OB: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OA, sa, OB, sb);
  switch (oa * 4 + ob) {
    SVDQ_MX_CASE(0, 0) SVDQ_MX_CASE(0, 1) SVDQ_MX_CASE(0, 2) SVDQ_MX_CASE(0, 3)
    SVDQ_MX_CASE(1, 0) SVDQ_MX_CASE(1, 1) SVDQ_MX_CASE(1, 2) SVDQ_MX_CASE(1, 3)
    SVDQ_MX_CASE(2, 0) SVDQ_MX_CASE(2, 1) SVDQ_MX_CASE(2, 2) SVDQ_MX_CASE(2, 3)
    SVDQ_MX_CASE(3, 0) SVDQ_MX_CASE(3, 1) SVDQ_MX_CASE(3, 2) SVDQ_MX_CASE(3, 3)
    default: return c;
  }
#undef SVDQ_MX_CASE
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* glb_ptr_t;

__device__ __forceinline__ void lds_load16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)g, (lds_ptr_t)l, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)g, (lds_ptr_t)l, 4, 0, 0);
}

// s_waitcnt vmcnt(n) leaving expcnt and lgkmcnt unconstrained
#define SVDQ_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8))
// s_waitcnt lgkmcnt(0) leaving vmcnt and expcnt unconstrained
#define SVDQ_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (0x7 << 4))

template <int DT, bool GELU>
__global__ __launch_bounds__(256) void k2_mx(MxParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[mx::STAGES * mx::STAGE_BYTES];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;

  // XCD-aware tile index: workgroups are dealt to the 8 XCDs round robin, so
  // give XCD x a contiguous range of the tile order.
  const int T = p.tiles_n * p.tiles_m;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, kx = bid >> 3, per = T >> 3, rem = T & 7;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int gsz_full = mx::GROUP_M * p.tiles_n;
  const int grp = tile / gsz_full, first_m = grp * mx::GROUP_M;
  const int gm = (p.tiles_m - first_m) < mx::GROUP_M ? (p.tiles_m - first_m) : mx::GROUP_M;
  const int within = tile - grp * gsz_full;
  const int tm = first_m + within % gm, tn = within / gm;
  const int64_t n0 = int64_t(tn) * 256, m0 = int64_t(tm) * 256;
  const int nsteps = int(p.K / KSTEP);
  const int64_t nfr = p.N / 16;            // valid weight fragment rows

  // this wave's share of every stage: weight frags 4w..4w+3, activation
  // frags 4w..4w+3, scale group w of each operand
  const uint8_t* ga[4];
  const uint8_t* gb[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    int64_t nt = n0 / 16 + 4 * wave + f;
    nt = nt < nfr ? nt : nfr - 1;            // a partial last tile re-reads a valid fragment
    ga[f] = p.wq + (nt * nsteps) * 1024 + lane * 16;
    gb[f] = p.xq + ((m0 / 16 + 4 * wave + f) * nsteps) * 1024 + lane * 16;
  }
  int64_t sgn = n0 / 64 + wave;
  sgn = sgn < p.N / 64 ? sgn : p.N / 64 - 1;
  const uint8_t* gsa = p.sw + (sgn * nsteps) * 256 + lane * 4;
  const uint8_t* gsb = p.sx + ((m0 / 64 + wave) * nsteps) * 256 + lane * 4;

  auto issue = [&](int s, int st) {
    uint8_t* base = smem + st * mx::STAGE_BYTES;
#pragma unroll
    for (int f = 0; f < 4; ++f) lds_load16(ga[f] + int64_t(s) * 1024, base + mx::A_OFF + (4 * wave + f) * 1024);
#pragma unroll
    for (int f = 0; f < 4; ++f) lds_load16(gb[f] + int64_t(s) * 1024, base + mx::B_OFF + (4 * wave + f) * 1024);
    lds_load4(gsa + int64_t(s) * 256, base + mx::SA_OFF + wave * 256);
    lds_load4(gsb + int64_t(s) * 256, base + mx::SB_OFF + wave * 256);
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragments of one step in registers (double-buffered across steps)
  struct Frags {
    u32x4 a[8], b[8];
    int sa0, sa1, sb0, sb1;
  };
  auto read_frags = [&](Frags& F, int st) {
    const uint8_t* base = smem + st * mx::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < 8; ++j) F.b[j] = *reinterpret_cast<const u32x4*>(base + mx::B_OFF + (8 * wm + j) * 1024 + lane * 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) F.a[i] = *reinterpret_cast<const u32x4*>(base + mx::A_OFF + (8 * wn + i) * 1024 + lane * 16);
    F.sb0 = *reinterpret_cast<const int*>(base + mx::SB_OFF + (2 * wm) * 256 + lane * 4);
    F.sb1 = *reinterpret_cast<const int*>(base + mx::SB_OFF + (2 * wm + 1) * 256 + lane * 4);
    F.sa0 = *reinterpret_cast<const int*>(base + mx::SA_OFF + (2 * wn) * 256 + lane * 4);
    F.sa1 = *reinterpret_cast<const int*>(base + mx::SA_OFF + (2 * wn + 1) * 256 + lane * 4);
  };
  auto compute = [&](const Frags& F) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const i32x8 a = i32x8{int(F.a[i][0]), int(F.a[i][1]), int(F.a[i][2]), int(F.a[i][3]), 0, 0, 0, 0};
      const int sa = i < 4 ? F.sa0 : F.sa1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const i32x8 b = i32x8{int(F.b[j][0]), int(F.b[j][1]), int(F.b[j][2]), int(F.b[j][3]), 0, 0, 0, 0};
        const int sb = j < 4 ? F.sb0 : F.sb1;
        acc[i][j] = mfma_mx(a, b, acc[i][j], sa, sb, i & 3, j & 3);
      }
    }
  };
  // Iteration s: wait until step s+1 is in LDS (its own loads, then the
  // barrier for everyone's), refill the stage step s-1 used with step s+3,
  // start reading step s+1's fragments, and run step s's 64 MFMAs meanwhile.
  auto body = [&](int s, Frags& cur, Frags& nxt) {
    // cur's LDS reads were issued an iteration ago; retire them here so the
    // 18 reads below need no counter slot (lgkmcnt counts at most 15)
    SVDQ_WAIT_LGKM0();
    if (s + 1 < nsteps) {
      if (s + 2 < nsteps) SVDQ_WAIT_VM(10);
      else SVDQ_WAIT_VM(0);
      __builtin_amdgcn_s_barrier();
      if (s + mx::STAGES - 1 < nsteps) issue(s + mx::STAGES - 1, (s + mx::STAGES - 1) % mx::STAGES);
      read_frags(nxt, (s + 1) % mx::STAGES);
    }
    compute(cur);
  };

#pragma unroll
  for (int s = 0; s < mx::STAGES - 1; ++s)
    if (s < nsteps) issue(s, s);
  if (nsteps > 2) SVDQ_WAIT_VM(20);
  else if (nsteps > 1) SVDQ_WAIT_VM(10);
  else SVDQ_WAIT_VM(0);
  __builtin_amdgcn_s_barrier();
  Frags F0, F1;
  read_frags(F0, 0);
  for (int s = 0; s < nsteps; s += 2) {
    body(s, F0, F1);
    if (s + 1 < nsteps) body(s + 1, F1, F0);
  }

  // epilogue: + T L2 (16-bit MFMA), + bias, GELU, round, store
  const u32x4* l2 = reinterpret_cast<const u32x4*>(p.l2);
  const u32x4* tt = reinterpret_cast<const u32x4*>(p.t);
  const int64_t ntw = n0 / 16 + 8 * wn, mtw = m0 / 16 + 8 * wm;
  for (int c = 0; c < p.nchunks; ++c) {
    u32x4 tb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) tb[j] = tt[((mtw + j) * (p.slots / 32) + c) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t nt = ntw + i;
      nt = nt < nfr ? nt : nfr - 1;
      const u32x4 la = l2[(nt * (p.slots / 32) + c) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mfma16<DT>(la, tb[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = n0 + 128 * wn + 16 * i + 4 * q;
    if (n >= p.N) continue;
    const f32x4 bv = *reinterpret_cast<const f32x4*>(p.bias + n);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t m = m0 + 128 * wm + 16 * j + (lane & 15);
      if (m < p.M) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][j][r] + bv[r];
          if constexpr (GELU) v[r] = gelu_erf(v[r]);
        }
        const unsigned lo = f2h<DT>(v[0]) | (f2h<DT>(v[1]) << 16);
        const unsigned hi = f2h<DT>(v[2]) | (f2h<DT>(v[3]) << 16);
        *reinterpret_cast<u32x2*>(p.Y + m * p.ldy + n) = u32x2{lo, hi};
      }
    }
  }
}

// -------------------------------------------------- INT4 per-group products
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

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <int FMT, int DT>
void launch_k1(const K1Params& kp, int64_t Mp, hipStream_t st) {
  hipLaunchKernelGGL((k1_act<FMT, DT>), dim3(unsigned(Mp / 16)), dim3(256), 0, st, kp);
}

template <int DT>
void launch_k2_int4(const K2Params& kp, int64_t Mp, bool gelu, hipStream_t st) {
  dim3 grid(unsigned(kp.N / 128), unsigned(Mp / 128));
  if (gelu) hipLaunchKernelGGL((k2_int4<DT, true>), grid, dim3(256), 0, st, kp);
  else hipLaunchKernelGGL((k2_int4<DT, false>), grid, dim3(256), 0, st, kp);
}

template <int DT>
void launch_k2_mx(const K2Params& kp, int64_t Mp, bool gelu, hipStream_t st) {
  MxParams mp;
  mp.wq = kp.wq; mp.sw = kp.sw; mp.l2 = kp.l2; mp.bias = kp.bias; mp.xq = kp.xq; mp.sx = kp.sx; mp.t = kp.t;
  mp.Y = kp.Y; mp.ldy = kp.ldy; mp.M = kp.M; mp.N = kp.N; mp.K = kp.K; mp.slots = kp.slots; mp.nchunks = kp.nchunks;
  mp.tiles_n = int(svdq::ceil_div(kp.N, 256));
  mp.tiles_m = int(Mp / 256);
  dim3 grid(unsigned(mp.tiles_n * mp.tiles_m));
  if (gelu) hipLaunchKernelGGL((k2_mx<DT, true>), grid, dim3(256), 0, st, mp);
  else hipLaunchKernelGGL((k2_mx<DT, false>), grid, dim3(256), 0, st, mp);
}

svdq_status check_device_layer(const svdq_layer* L) {
  svdq_status s = svdq::validate_layer(L);
  if (s != SVDQ_OK) return s;
  if (!L->blob_on_device) return SVDQ_ERR_INVALID_ARG;
  if (!aligned(L->blob, 256)) return SVDQ_ERR_INVALID_ARG;
  return SVDQ_OK;
}

}  // namespace

extern "C" svdq_status svdq_quantize_activations(const svdq_layer* L, const void* X_dev, int64_t M, int64_t ldx,
                                                 void* ws_dev, size_t ws_bytes, hipStream_t stream) {
  svdq_status st = check_device_layer(L);
  if (st != SVDQ_OK) return st;
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  if (!X_dev || !ws_dev) return SVDQ_ERR_INVALID_ARG;
  if (ldx < L->K || ldx % 8 != 0 || !aligned(X_dev, 16)) return SVDQ_ERR_SHAPE;
  svdq::WsOffsets w = svdq::ws_offsets(M, L->K, L->rank_slots, L->fmt);
  if (ws_bytes < w.total) return SVDQ_ERR_CAPACITY;
  if (!aligned(ws_dev, 256)) return SVDQ_ERR_INVALID_ARG;
  const uint8_t* blob = static_cast<const uint8_t*>(L->blob);
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  K1Params kp;
  kp.X = static_cast<const uint16_t*>(X_dev);
  kp.ldx = ldx; kp.M = M; kp.K = L->K;
  kp.invlam = reinterpret_cast<const float*>(blob + L->off_invlam);
  kp.l1x = reinterpret_cast<const uint16_t*>(blob + L->off_l1x);
  kp.slots = L->rank_slots;
  kp.njt = 2 * int(svdq::ceil_div(L->rank_active, 32));
  kp.xq = ws + w.xq; kp.sx = ws + w.sx; kp.t = reinterpret_cast<uint16_t*>(ws + w.t);
  if (L->fmt == SVDQ_FMT_INT4_G64) {
    if (L->dtype == SVDQ_BF16) launch_k1<SVDQ_FMT_INT4_G64, SVDQ_BF16>(kp, w.Mp, stream);
    else launch_k1<SVDQ_FMT_INT4_G64, SVDQ_F16>(kp, w.Mp, stream);
  } else {
    if (L->dtype == SVDQ_BF16) launch_k1<SVDQ_FMT_MXFP4_G32, SVDQ_BF16>(kp, w.Mp, stream);
    else launch_k1<SVDQ_FMT_MXFP4_G32, SVDQ_F16>(kp, w.Mp, stream);
  }
  return launch_ok();
}

extern "C" svdq_status svdq_gemm_forward(const svdq_layer* L, int64_t M, void* Y_dev, int64_t ldy,
                                         const void* ws_dev, size_t ws_bytes, unsigned flags, hipStream_t stream) {
  svdq_status st = check_device_layer(L);
  if (st != SVDQ_OK) return st;
  if (M < 0 || (flags & ~unsigned(SVDQ_FLAG_GELU)) != 0u) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  if (!Y_dev || !ws_dev) return SVDQ_ERR_INVALID_ARG;
  if (ldy < L->N || ldy % 4 != 0 || !aligned(Y_dev, 8)) return SVDQ_ERR_SHAPE;
  svdq::WsOffsets w = svdq::ws_offsets(M, L->K, L->rank_slots, L->fmt);
  if (ws_bytes < w.total) return SVDQ_ERR_CAPACITY;
  if (!aligned(ws_dev, 256)) return SVDQ_ERR_INVALID_ARG;
  const uint8_t* blob = static_cast<const uint8_t*>(L->blob);
  const uint8_t* ws = static_cast<const uint8_t*>(ws_dev);
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
  kp.nchunks = int(svdq::ceil_div(L->rank_active, 32));
  const bool gelu = (flags & SVDQ_FLAG_GELU) != 0u;
  if (L->fmt == SVDQ_FMT_INT4_G64) {
    if (L->dtype == SVDQ_BF16) launch_k2_int4<SVDQ_BF16>(kp, w.Mp, gelu, stream);
    else launch_k2_int4<SVDQ_F16>(kp, w.Mp, gelu, stream);
  } else {
    if (L->dtype == SVDQ_BF16) launch_k2_mx<SVDQ_BF16>(kp, w.Mp, gelu, stream);
    else launch_k2_mx<SVDQ_F16>(kp, w.Mp, gelu, stream);
  }
  return launch_ok();
}

extern "C" svdq_status svdq_linear_forward(const svdq_layer* L, const void* X_dev, int64_t M, int64_t ldx,
                                           void* Y_dev, int64_t ldy, void* ws_dev, size_t ws_bytes, unsigned flags,
                                           hipStream_t stream) {
  svdq_status st = check_device_layer(L);
  if (st != SVDQ_OK) return st;
  if (M < 0 || (flags & ~unsigned(SVDQ_FLAG_GELU)) != 0u) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  if (!Y_dev) return SVDQ_ERR_INVALID_ARG;
  if (ldy < L->N || ldy % 4 != 0 || !aligned(Y_dev, 8)) return SVDQ_ERR_SHAPE;
  st = svdq_quantize_activations(L, X_dev, M, ldx, ws_dev, ws_bytes, stream);
  if (st != SVDQ_OK) return st;
  return svdq_gemm_forward(L, M, Y_dev, ldy, ws_dev, ws_bytes, flags, stream);
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
