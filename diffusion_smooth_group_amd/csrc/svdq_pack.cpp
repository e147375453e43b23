// svdq_pack.cpp -- offline pack, LoRA attach and the inspection exports of
// the C ABI (include/svdq.h).  Host code; the only device interaction is
// copying the finished blob.
//
// SVDQuant paper ("SVDQuant: Absorbing Outliers by Low-Rank Components for
// 4-Bit Diffusion Models"): smoothing §4.2 / Fig. 4, low-rank split §4.2 /
// Eq. 5 / Fig. 5, quantizer §3, group sizes and scale types §5.1
// (implementation details), LoRA in the low-rank branch §5.2.
//
// This translation unit is compiled with -ffp-contract=off: the residual and
// the quantizers must round exactly as written.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <vector>

#include "svdq.h"
#include "svdq_host.h"
#include "svdq_layout.h"

using namespace svdq;

extern "C" const char* svdq_status_string(svdq_status s) {
  switch (s) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_INVALID_ARG: return "invalid argument";
    case SVDQ_ERR_SHAPE: return "unsupported or inconsistent shape";
    case SVDQ_ERR_UNSUPPORTED: return "unsupported request";
    case SVDQ_ERR_CAPACITY: return "capacity exceeded";
    case SVDQ_ERR_NUMERIC: return "non-finite input";
    case SVDQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

namespace {

int slots_for(int capacity) { return int(round_up(std::max(capacity, 0), 32)); }

svdq_status check_common(int64_t K, int64_t N, int rank_capacity, int fmt, int dtype) {
  if (fmt != SVDQ_FMT_INT4_G64 && fmt != SVDQ_FMT_MXFP4_G32 && fmt != SVDQ_FMT_INT8_W8A8) return SVDQ_ERR_INVALID_ARG;
  if (dtype != SVDQ_F16 && dtype != SVDQ_BF16) return SVDQ_ERR_INVALID_ARG;
  if (K <= 0 || N <= 0) return SVDQ_ERR_SHAPE;
  if (K % KSTEP != 0 || N % 128 != 0) return SVDQ_ERR_SHAPE;
  if (rank_capacity < 0 || rank_capacity > SVDQ_MAX_RANK_CAPACITY) return SVDQ_ERR_INVALID_ARG;
  return SVDQ_OK;
}

void fill_layer(svdq_layer* L, int64_t K, int64_t N, int rank, int rank_active, int capacity, int fmt,
                int dtype, int has_bias, int on_dev, void* blob, size_t bytes) {
  BlobOffsets o = blob_offsets(K, N, slots_for(capacity), fmt);
  std::memset(L, 0, sizeof(*L));
  L->K = K; L->N = N; L->rank = rank; L->rank_active = rank_active; L->rank_capacity = capacity;
  L->rank_slots = slots_for(capacity); L->fmt = fmt; L->dtype = dtype; L->has_bias = has_bias;
  L->blob_on_device = on_dev; L->blob = blob; L->blob_bytes = bytes;
  L->off_invlam = o.invlam; L->off_lam = o.lam; L->off_l1x = o.l1x; L->off_l2 = o.l2;
  L->off_wq = o.wq; L->off_sw = o.sw; L->off_bias = o.bias;
}

void write_header(uint8_t* blob, const svdq_layer& L) {
  BlobHeader h;
  std::memset(&h, 0, sizeof(h));
  h.magic = BLOB_MAGIC; h.version = BLOB_VERSION; h.K = L.K; h.N = L.N;
  h.rank = L.rank; h.rank_active = L.rank_active; h.rank_capacity = L.rank_capacity;
  h.rank_slots = L.rank_slots; h.fmt = L.fmt; h.dtype = L.dtype; h.has_bias = L.has_bias;
  BlobOffsets o = blob_offsets(L.K, L.N, L.rank_slots, L.fmt);
  h.off_invlam = o.invlam; h.off_lam = o.lam; h.off_l1x = o.l1x; h.off_l2 = o.l2; h.off_wq = o.wq;
  h.off_sw = o.sw; h.off_bias = o.bias; h.total = o.total;
  std::memset(blob, 0, HDR_BYTES);
  std::memcpy(blob, &h, sizeof(h));
}

}  // namespace

namespace svdq {
svdq_status validate_layer(const svdq_layer* L) {
  if (!L || !L->blob) return SVDQ_ERR_INVALID_ARG;
  svdq_status st = check_common(L->K, L->N, L->rank_capacity, L->fmt, L->dtype);
  if (st != SVDQ_OK) return st;
  if (L->rank < 0 || L->rank_active < L->rank || L->rank_active > L->rank_capacity) return SVDQ_ERR_INVALID_ARG;
  if (L->rank_slots != slots_for(L->rank_capacity)) return SVDQ_ERR_INVALID_ARG;
  BlobOffsets o = blob_offsets(L->K, L->N, L->rank_slots, L->fmt);
  if (L->blob_bytes < o.total) return SVDQ_ERR_CAPACITY;
  if (L->off_wq != o.wq || L->off_l1x != o.l1x || L->off_l2 != o.l2 || L->off_sw != o.sw ||
      L->off_bias != o.bias || L->off_invlam != o.invlam || L->off_lam != o.lam)
    return SVDQ_ERR_INVALID_ARG;
  return SVDQ_OK;
}
}  // namespace svdq

namespace {

// Core pack into a host byte buffer.
svdq_status pack_host(const void* W_host, int64_t K, int64_t N, int64_t ldw, int dtype, const float* absmax,
                      int rank, int capacity, int fmt, const void* bias_host, uint8_t* blob, size_t bytes,
                      svdq_layer* out, int on_dev, void* blob_ptr_for_desc, int refine_iters = 0,
                      double* errors = nullptr) {
  svdq_status st = check_common(K, N, capacity, fmt, dtype);
  if (st != SVDQ_OK) return st;
  if (!W_host || !out) return SVDQ_ERR_INVALID_ARG;
  if (ldw < N) return SVDQ_ERR_SHAPE;
  if (rank < 0 || rank > capacity || rank > std::min(K, N)) return SVDQ_ERR_INVALID_ARG;
  if (refine_iters < 0 || refine_iters > SVDQ_MAX_REFINE_ITERS) return SVDQ_ERR_INVALID_ARG;
  const int slots = slots_for(capacity);
  BlobOffsets o = blob_offsets(K, N, slots, fmt);
  if (!blob || bytes < o.total) return SVDQ_ERR_CAPACITY;

  const uint16_t* Wb = static_cast<const uint16_t*>(W_host);
  std::vector<float> W(size_t(K) * N);
  std::vector<float> wmax(K, 0.0f);
  std::atomic<bool> finite(true);
  parallel_for(K, [&](int64_t b, int64_t e) {
    for (int64_t j = b; j < e; ++j) {
      float m = 0.0f;
      for (int64_t n = 0; n < N; ++n) {
        float v = h16_to_f32(Wb[j * ldw + n], dtype);
        W[size_t(j) * N + n] = v;
        if (!std::isfinite(v)) finite.store(false, std::memory_order_relaxed);
        m = std::fmax(m, std::fabs(v));
      }
      wmax[j] = m;
    }
  });
  if (!finite.load()) return SVDQ_ERR_NUMERIC;
  // lambda_j = sqrt(a_j / w_j); 1 where either maximum is zero or the ratio
  // is not a positive finite fp32 number.
  std::vector<float> lam(K), invlam(K);
  for (int64_t j = 0; j < K; ++j) {
    float a = absmax ? absmax[j] : 0.0f;
    if (absmax && (!std::isfinite(a) || a < 0.0f)) return SVDQ_ERR_NUMERIC;
    float w = wmax[j];
    float l = 1.0f;
    if (a > 0.0f && w > 0.0f) {
      float ratio = a / w;
      float sq = std::sqrt(ratio);
      if (std::isfinite(ratio) && ratio > 0.0f && std::isfinite(sq) && sq > 0.0f) l = sq;
    }
    lam[j] = l;
    invlam[j] = 1.0f / l;
  }
  // One candidate split: 16-bit factors, the fp32 residual's codes and
  // scales per output column (canonical [N][K] / [N][K/G]), and its error.
  const bool i8 = fmt == SVDQ_FMT_INT8_W8A8;
  const int64_t G = i8 ? K : group_size(fmt);   // INT8: one scale per output channel
  const int rk = std::max(rank, 1);
  struct Cand {
    std::vector<uint16_t> l1x, l2q;   // K x rank, rank x N
    std::vector<uint8_t> q;           // INT4 / INT8: int8 value; MXFP4: E2M1 code
    std::vector<uint16_t> sc;         // INT4: fp16 bits; MXFP4: e8m0
    std::vector<float> sf;            // INT8: fp32 channel scales
    double err = 0.0;
  };
  auto what = [&](int64_t j, int64_t n) { return double(lam[j]) * double(W[size_t(j) * N + n]); };
  // low-rank term at row j: s[n] = sum_k L1x[j,k] L2q[k,n], k ascending (float64)
  auto lowrank_row = [&](const Cand& c, int64_t j, std::vector<double>& srow, const std::vector<double>& l2d) {
    std::fill(srow.begin(), srow.end(), 0.0);
    for (int k = 0; k < rank; ++k) {
      double a = h16_to_f32(c.l1x[size_t(j) * rank + k], dtype);
      const double* l2r = &l2d[size_t(k) * N];
      for (int64_t n = 0; n < N; ++n) srow[n] = srow[n] + a * l2r[n];
    }
  };
  auto l2_double = [&](const Cand& c) {
    std::vector<double> l2d(size_t(rk) * N, 0.0);
    for (size_t i = 0; i < size_t(rank) * N; ++i) l2d[i] = h16_to_f32(c.l2q[i], dtype);
    return l2d;
  };
  auto deq = [&](const Cand& c, int64_t n, int64_t k) -> double {
    if (i8) return double(int8_t(c.q[size_t(n) * K + k])) * double(c.sf[size_t(n)]);
    const size_t gi = size_t(n) * (K / G) + size_t(k / G);
    if (fmt == SVDQ_FMT_INT4_G64)
      return double(int8_t(c.q[size_t(n) * K + k])) * double(f16_to_f32(c.sc[gi]));
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const uint8_t code = c.q[size_t(n) * K + k];
    const double v = grid[code & 7] * std::ldexp(1.0, int(c.sc[gi]) - 127);
    return (code & 8) ? -v : v;
  };
  // factors of the split of matrix B (K x N, float64), rounded to 16 bits
  auto factors = [&](const std::vector<double>& B, Cand& c) -> bool {
    c.l1x.assign(size_t(K) * rk, 0);
    c.l2q.assign(size_t(rk) * N, 0);
    if (rank == 0) return true;
    std::vector<double> L1(size_t(K) * rank), L2(size_t(rank) * N);
    if (!truncated_svd(B.data(), K, N, rank, L1.data(), L2.data(), nullptr)) return false;
    for (int64_t j = 0; j < K; ++j)
      for (int i = 0; i < rank; ++i)
        c.l1x[size_t(j) * rank + i] = f64_to_h16_rne(double(invlam[j]) * L1[size_t(j) * rank + i], dtype);
    for (size_t i = 0; i < size_t(rank) * N; ++i) c.l2q[i] = f64_to_h16_rne(L2[i], dtype);
    return true;
  };
  // R = fl32(lambda W - lambda * sum_k L1x[:,k] L2q[k,:]), its group codes
  // (per output column, groups along K), and the split's error
  // ||W_hat - diag(lambda) L1x L2q - deq(Q(R))||_F^2 in float64
  auto residual_codes = [&](Cand& c) {
    std::vector<float> Rt(size_t(N) * K);
    const std::vector<double> l2d = l2_double(c);
    parallel_for(K, [&](int64_t b, int64_t e) {
      std::vector<double> srow(N);
      for (int64_t j = b; j < e; ++j) {
        lowrank_row(c, j, srow, l2d);
        const double lj = double(lam[j]);
        for (int64_t n = 0; n < N; ++n) Rt[size_t(n) * K + j] = float(what(j, n) - lj * srow[n]);
      }
    });
    c.q.assign(size_t(N) * K, 0);
    c.sc.assign(size_t(N) * (K / G), 0);
    if (i8) c.sf.assign(size_t(N), 0.0f);
    parallel_for(N, [&](int64_t nb, int64_t ne) {
      std::vector<int8_t> qi(i8 ? size_t(K) : 64);
      std::vector<uint8_t> qm(32);
      for (int64_t n = nb; n < ne; ++n)
        for (int64_t g = 0; g < K / G; ++g) {
          const float* v = &Rt[size_t(n) * K + g * G];
          uint8_t* qo = &c.q[size_t(n) * K + g * G];
          if (i8) {
            quant_int8_row(v, K, qi.data(), &c.sf[size_t(n)]);
            for (int64_t i = 0; i < K; ++i) qo[i] = uint8_t(qi[i]);
          } else if (fmt == SVDQ_FMT_INT4_G64) {
            uint16_t sbits;
            quant_int4_group(v, qi.data(), &sbits);
            c.sc[size_t(n) * (K / G) + g] = sbits;
            for (int i = 0; i < G; ++i) qo[i] = uint8_t(qi[i]);
          } else {
            uint8_t e;
            quant_mx_group(v, qm.data(), &e);
            c.sc[size_t(n) * (K / G) + g] = e;
            for (int i = 0; i < G; ++i) qo[i] = qm[i];
          }
        }
    });
    std::vector<double> part(size_t(K), 0.0);
    parallel_for(K, [&](int64_t b, int64_t e) {
      std::vector<double> srow(N);
      for (int64_t j = b; j < e; ++j) {
        lowrank_row(c, j, srow, l2d);
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double d = what(j, n) - double(lam[j]) * srow[n] - deq(c, n, j);
          acc += d * d;
        }
        part[j] = acc;
      }
    });
    c.err = 0.0;
    for (int64_t j = 0; j < K; ++j) c.err += part[j];
  };

  // one-shot split of W_hat = diag(lambda) W (exact in float64) [SVDQuant
  // §4.2], then refine_iters rounds that split W_hat - deq(Q(R)) again and
  // re-derive R; the split with the smallest error is kept
  Cand best;
  {
    std::vector<double> A;
    if (rank > 0) {
      A.resize(size_t(K) * N);
      parallel_for(K, [&](int64_t b, int64_t e) {
        for (int64_t j = b; j < e; ++j)
          for (int64_t n = 0; n < N; ++n) A[size_t(j) * N + n] = what(j, n);
      });
    }
    if (!factors(A, best)) return SVDQ_ERR_NUMERIC;
    residual_codes(best);
    if (errors) errors[0] = best.err;
    Cand cur = best;
    for (int it = 1; it <= refine_iters && rank > 0; ++it) {
      parallel_for(K, [&](int64_t b, int64_t e) {
        for (int64_t j = b; j < e; ++j)
          for (int64_t n = 0; n < N; ++n) A[size_t(j) * N + n] = what(j, n) - deq(cur, n, j);
      });
      Cand next;
      if (!factors(A, next)) return SVDQ_ERR_NUMERIC;
      residual_codes(next);
      if (errors) errors[it] = next.err;
      cur = std::move(next);
      if (cur.err < best.err) best = cur;
    }
  }
  std::memset(blob, 0, o.total);
  // residual codes and scales, tiled
  uint8_t* wq = blob + o.wq;
  uint8_t* sw = blob + o.sw;
  parallel_for(N / 16, [&](int64_t tb, int64_t te) {
    for (int64_t n = tb * 16; n < te * 16; ++n)
      for (int64_t g = 0; g < K / G; ++g) {
        const uint16_t sv = best.sc[size_t(n) * (K / G) + g];
        if (i8) std::memcpy(sw + 4 * n, &best.sf[size_t(n)], 4);
        else if (fmt == SVDQ_FMT_INT4_G64) std::memcpy(sw + 2 * int4_wscale_pos(n, g, K), &sv, 2);
        else sw[mx_scale_pos(n, g, K)] = uint8_t(sv);
        for (int64_t i = 0; i < G; ++i) {
          size_t byte; int nib;
          code_pos(n, g * G + i, K, fmt, &byte, &nib);
          const uint8_t c = best.q[size_t(n) * K + g * G + i];
          wq[byte] |= i8 ? c : uint8_t((c & 0xF) << (4 * nib));
        }
      }
  });
  const std::vector<uint16_t>& l1x = best.l1x;
  const std::vector<uint16_t>& l2q = best.l2q;
  // factors, tiled
  uint16_t* l1t = reinterpret_cast<uint16_t*>(blob + o.l1x);
  uint16_t* l2t = reinterpret_cast<uint16_t*>(blob + o.l2);
  for (int64_t j = 0; j < K; ++j)
    for (int i = 0; i < rank; ++i) l1t[l1x_pos(j, i, slots, fmt)] = l1x[size_t(j) * rank + i];
  for (int i = 0; i < rank; ++i)
    for (int64_t n = 0; n < N; ++n) l2t[lr_pos(n, i, slots, fmt)] = l2q[size_t(i) * N + n];
  std::memcpy(blob + o.invlam, invlam.data(), size_t(K) * 4);
  std::memcpy(blob + o.lam, lam.data(), size_t(K) * 4);
  float* bias = reinterpret_cast<float*>(blob + o.bias);
  if (bias_host) {
    const uint16_t* bb = static_cast<const uint16_t*>(bias_host);
    for (int64_t n = 0; n < N; ++n) bias[n] = h16_to_f32(bb[n], dtype);
  }
  fill_layer(out, K, N, rank, rank, capacity, fmt, dtype, bias_host ? 1 : 0, on_dev, blob_ptr_for_desc, bytes);
  write_header(blob, *out);
  return SVDQ_OK;
}

svdq_status copy_bytes(void* dst, int dst_dev, const void* src, int src_dev, size_t n, hipStream_t stream) {
  if (n == 0) return SVDQ_OK;
  if (!dst_dev && !src_dev) { std::memcpy(dst, src, n); return SVDQ_OK; }
  hipMemcpyKind kind = dst_dev ? (src_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice)
                               : hipMemcpyDeviceToHost;
  if (hipMemcpyAsync(dst, src, n, kind, stream) != hipSuccess) return SVDQ_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SVDQ_ERR_HIP;
  return SVDQ_OK;
}

// Host view of a layer's blob (copied from the device when needed).
svdq_status host_blob(const svdq_layer* L, std::vector<uint8_t>& tmp, const uint8_t** view, hipStream_t stream) {
  if (!L->blob_on_device) { *view = static_cast<const uint8_t*>(L->blob); return SVDQ_OK; }
  BlobOffsets o = blob_offsets(L->K, L->N, L->rank_slots, L->fmt);
  tmp.resize(o.total);
  svdq_status st = copy_bytes(tmp.data(), 0, L->blob, 1, o.total, stream);
  *view = tmp.data();
  return st;
}

}  // namespace

extern "C" svdq_status svdq_packed_size(int64_t K, int64_t N, int rank_capacity, svdq_format fmt,
                                        svdq_dtype dtype, size_t* bytes) {
  svdq_status st = check_common(K, N, rank_capacity, fmt, dtype);
  if (st != SVDQ_OK) return st;
  if (!bytes) return SVDQ_ERR_INVALID_ARG;
  *bytes = blob_offsets(K, N, slots_for(rank_capacity), fmt).total;
  return SVDQ_OK;
}

extern "C" svdq_status svdq_pack_weights_host(const void* W_host, int64_t K, int64_t N, int64_t ldw,
                                              svdq_dtype dtype, const float* act_absmax_host, int rank,
                                              int rank_capacity, svdq_format fmt, const void* bias_host,
                                              void* blob_host, size_t blob_bytes, svdq_layer* out) {
  return pack_host(W_host, K, N, ldw, dtype, act_absmax_host, rank, rank_capacity, fmt, bias_host,
                   static_cast<uint8_t*>(blob_host), blob_bytes, out, 0, blob_host);
}

extern "C" svdq_status svdq_pack_weights(const void* W_host, int64_t K, int64_t N, int64_t ldw, svdq_dtype dtype,
                                         const float* act_absmax_host, int rank, int rank_capacity,
                                         svdq_format fmt, const void* bias_host, void* blob_dev, size_t blob_bytes,
                                         hipStream_t stream, svdq_layer* out) {
  svdq_status st = check_common(K, N, rank_capacity, fmt, dtype);
  if (st != SVDQ_OK) return st;
  if (!blob_dev || !out) return SVDQ_ERR_INVALID_ARG;
  size_t need = blob_offsets(K, N, slots_for(rank_capacity), fmt).total;
  if (blob_bytes < need) return SVDQ_ERR_CAPACITY;
  std::vector<uint8_t> host(need);
  st = pack_host(W_host, K, N, ldw, dtype, act_absmax_host, rank, rank_capacity, fmt, bias_host, host.data(),
                 need, out, 1, blob_dev);
  if (st != SVDQ_OK) return st;
  out->blob_bytes = blob_bytes;
  return copy_bytes(blob_dev, 1, host.data(), 0, need, stream);
}

extern "C" svdq_status svdq_pack_weights_ex(const void* W_host, int64_t K, int64_t N, int64_t ldw, svdq_dtype dtype,
                                            const float* act_absmax_host, int rank, int rank_capacity,
                                            svdq_format fmt, const void* bias_host, int refine_iters,
                                            double* errors_out, void* blob, size_t blob_bytes, int blob_on_device,
                                            hipStream_t stream, svdq_layer* out) {
  svdq_status st = check_common(K, N, rank_capacity, fmt, dtype);
  if (st != SVDQ_OK) return st;
  if (!blob || !out) return SVDQ_ERR_INVALID_ARG;
  size_t need = blob_offsets(K, N, slots_for(rank_capacity), fmt).total;
  if (blob_bytes < need) return SVDQ_ERR_CAPACITY;
  if (!blob_on_device)
    return pack_host(W_host, K, N, ldw, dtype, act_absmax_host, rank, rank_capacity, fmt, bias_host,
                     static_cast<uint8_t*>(blob), blob_bytes, out, 0, blob, refine_iters, errors_out);
  std::vector<uint8_t> host(need);
  st = pack_host(W_host, K, N, ldw, dtype, act_absmax_host, rank, rank_capacity, fmt, bias_host, host.data(),
                 need, out, 1, blob, refine_iters, errors_out);
  if (st != SVDQ_OK) return st;
  out->blob_bytes = blob_bytes;
  return copy_bytes(blob, 1, host.data(), 0, need, stream);
}

extern "C" svdq_status svdq_layer_copy(const svdq_layer* src, void* dst, size_t dst_bytes, int dst_on_device,
                                       hipStream_t stream, svdq_layer* out) {
  svdq_status st = validate_layer(src);
  if (st != SVDQ_OK) return st;
  if (!dst || !out) return SVDQ_ERR_INVALID_ARG;
  size_t need = blob_offsets(src->K, src->N, src->rank_slots, src->fmt).total;
  if (dst_bytes < need) return SVDQ_ERR_CAPACITY;
  st = copy_bytes(dst, dst_on_device ? 1 : 0, src->blob, src->blob_on_device, need, stream);
  if (st != SVDQ_OK) return st;
  svdq_layer L = *src;
  L.blob = dst; L.blob_bytes = dst_bytes; L.blob_on_device = dst_on_device ? 1 : 0;
  *out = L;
  return SVDQ_OK;
}

namespace {
svdq_status write_lora(svdq_layer* L, const uint16_t* A, const uint16_t* B, int rL, float alpha,
                       hipStream_t stream) {
  std::vector<uint8_t> tmp;
  const uint8_t* view = nullptr;
  svdq_status st = host_blob(L, tmp, &view, stream);
  if (st != SVDQ_OK) return st;
  BlobOffsets o = blob_offsets(L->K, L->N, L->rank_slots, L->fmt);
  // edit a private copy of the two factor regions and the header
  std::vector<uint8_t> l1(view + o.l1x, view + o.l1x + size_t(L->K) * L->rank_slots * 2);
  std::vector<uint8_t> l2(view + o.l2, view + o.l2 + size_t(L->rank_slots) * L->N * 2);
  uint16_t* l1t = reinterpret_cast<uint16_t*>(l1.data());
  uint16_t* l2t = reinterpret_cast<uint16_t*>(l2.data());
  const int slots = L->rank_slots;
  for (int64_t k = 0; k < L->K; ++k)
    for (int j = L->rank; j < slots; ++j) {
      int i = j - L->rank;
      l1t[l1x_pos(k, j, slots, L->fmt)] = (i < rL) ? A[size_t(k) * rL + i] : uint16_t(0);
    }
  for (int j = L->rank; j < slots; ++j) {
    int i = j - L->rank;
    for (int64_t n = 0; n < L->N; ++n) {
      uint16_t v = 0;
      if (i < rL) v = f64_to_h16_rne(double(alpha) * double(h16_to_f32(B[size_t(i) * L->N + n], L->dtype)), L->dtype);
      l2t[lr_pos(n, j, slots, L->fmt)] = v;
    }
  }
  svdq_layer nl = *L;
  nl.rank_active = L->rank + rL;
  std::vector<uint8_t> hdr(HDR_BYTES);
  write_header(hdr.data(), nl);
  uint8_t* base = static_cast<uint8_t*>(L->blob);
  int dev = L->blob_on_device;
  if ((st = copy_bytes(base + o.l1x, dev, l1.data(), 0, l1.size(), stream)) != SVDQ_OK) return st;
  if ((st = copy_bytes(base + o.l2, dev, l2.data(), 0, l2.size(), stream)) != SVDQ_OK) return st;
  if ((st = copy_bytes(base, dev, hdr.data(), 0, HDR_BYTES, stream)) != SVDQ_OK) return st;
  L->rank_active = nl.rank_active;
  return SVDQ_OK;
}
}  // namespace

extern "C" svdq_status svdq_attach_lora(svdq_layer* layer, const void* A_host, const void* B_host, int rL,
                                        float alpha, hipStream_t stream) {
  svdq_status st = validate_layer(layer);
  if (st != SVDQ_OK) return st;
  if (!A_host || !B_host || rL <= 0 || !std::isfinite(alpha)) return SVDQ_ERR_INVALID_ARG;
  if (layer->rank + rL > layer->rank_capacity) return SVDQ_ERR_CAPACITY;
  return write_lora(layer, static_cast<const uint16_t*>(A_host), static_cast<const uint16_t*>(B_host), rL, alpha,
                    stream);
}

extern "C" svdq_status svdq_detach_lora(svdq_layer* layer, hipStream_t stream) {
  svdq_status st = validate_layer(layer);
  if (st != SVDQ_OK) return st;
  return write_lora(layer, nullptr, nullptr, 0, 1.0f, stream);
}

extern "C" svdq_status svdq_layer_export(const svdq_layer* L, float* lam, float* invlam, void* l1x, void* l2,
                                         void* codes, void* scales, float* bias, hipStream_t stream) {
  svdq_status st = validate_layer(L);
  if (st != SVDQ_OK) return st;
  std::vector<uint8_t> tmp;
  const uint8_t* v = nullptr;
  if ((st = host_blob(L, tmp, &v, stream)) != SVDQ_OK) return st;
  const int64_t K = L->K, N = L->N;
  const int slots = L->rank_slots, ra = L->rank_active;
  if (lam) std::memcpy(lam, v + L->off_lam, size_t(K) * 4);
  if (invlam) std::memcpy(invlam, v + L->off_invlam, size_t(K) * 4);
  if (bias) std::memcpy(bias, v + L->off_bias, size_t(N) * 4);
  const uint16_t* l1t = reinterpret_cast<const uint16_t*>(v + L->off_l1x);
  const uint16_t* l2t = reinterpret_cast<const uint16_t*>(v + L->off_l2);
  if (l1x) {
    uint16_t* o = static_cast<uint16_t*>(l1x);
    for (int64_t k = 0; k < K; ++k)
      for (int j = 0; j < ra; ++j) o[size_t(k) * ra + j] = l1t[l1x_pos(k, j, slots, L->fmt)];
  }
  if (l2) {
    uint16_t* o = static_cast<uint16_t*>(l2);
    for (int j = 0; j < ra; ++j)
      for (int64_t n = 0; n < N; ++n) o[size_t(j) * N + n] = l2t[lr_pos(n, j, slots, L->fmt)];
  }
  const uint8_t* wq = v + L->off_wq;
  if (codes) {
    uint8_t* o = static_cast<uint8_t*>(codes);
    parallel_for(K, [&](int64_t b, int64_t e) {
      for (int64_t k = b; k < e; ++k)
        for (int64_t n = 0; n < N; ++n) {
          size_t byte; int nib;
          code_pos(n, k, K, L->fmt, &byte, &nib);
          uint8_t c = L->fmt == SVDQ_FMT_INT8_W8A8 ? wq[byte] : uint8_t((wq[byte] >> (4 * nib)) & 0xF);
          if (L->fmt == SVDQ_FMT_INT4_G64) c = uint8_t(int8_t(uint8_t(c << 4)) >> 4);   // sign-extend
          o[size_t(k) * N + n] = c;
        }
    });
  }
  if (scales && L->fmt == SVDQ_FMT_INT8_W8A8) {
    std::memcpy(scales, v + L->off_sw, size_t(N) * 4);      // fp32 [1][N]
  } else if (scales) {
    const int G = group_size(L->fmt);
    for (int64_t g = 0; g < K / G; ++g)
      for (int64_t n = 0; n < N; ++n) {
        if (L->fmt == SVDQ_FMT_INT4_G64) {
          uint16_t s;
          std::memcpy(&s, v + L->off_sw + 2 * int4_wscale_pos(n, g, K), 2);
          static_cast<uint16_t*>(scales)[size_t(g) * N + n] = s;
        } else {
          static_cast<uint8_t*>(scales)[size_t(g) * N + n] = v[L->off_sw + mx_scale_pos(n, g, K)];
        }
      }
  }
  return SVDQ_OK;
}

extern "C" svdq_status svdq_workspace_size(const svdq_layer* layer, int64_t M, size_t* bytes) {
  svdq_status st = validate_layer(layer);
  if (st != SVDQ_OK) return st;
  if (!bytes || M < 0) return SVDQ_ERR_INVALID_ARG;
  *bytes = ws_offsets(M, layer->K, layer->rank_slots, layer->fmt).total;
  return SVDQ_OK;
}

extern "C" svdq_status svdq_workspace_export(const svdq_layer* L, const void* ws_dev, size_t ws_bytes, int64_t M,
                                             void* codes, void* scales, void* t, hipStream_t stream) {
  svdq_status st = validate_layer(L);
  if (st != SVDQ_OK) return st;
  if (!ws_dev || M < 0) return SVDQ_ERR_INVALID_ARG;
  const int64_t K = L->K;
  WsOffsets w = ws_offsets(M, K, L->rank_slots, L->fmt);
  if (ws_bytes < w.total) return SVDQ_ERR_CAPACITY;
  std::vector<uint8_t> h(w.total);
  if ((st = copy_bytes(h.data(), 0, ws_dev, 1, w.total, stream)) != SVDQ_OK) return st;
  const uint8_t* xq = h.data() + w.xq;
  if (codes) {
    uint8_t* o = static_cast<uint8_t*>(codes);
    parallel_for(M, [&](int64_t b, int64_t e) {
      for (int64_t m = b; m < e; ++m)
        for (int64_t k = 0; k < K; ++k) {
          size_t byte; int nib;
          code_pos(m, k, K, L->fmt, &byte, &nib);
          uint8_t c = L->fmt == SVDQ_FMT_INT8_W8A8 ? xq[byte] : uint8_t((xq[byte] >> (4 * nib)) & 0xF);
          if (L->fmt == SVDQ_FMT_INT4_G64) c = uint8_t(int8_t(uint8_t(c << 4)) >> 4);
          o[size_t(m) * K + k] = c;
        }
    });
  }
  if (scales && L->fmt == SVDQ_FMT_INT8_W8A8) {
    std::memcpy(scales, h.data() + w.sx, size_t(M) * 4);    // fp32 [M][1]
  } else if (scales) {
    const int G = group_size(L->fmt);
    for (int64_t m = 0; m < M; ++m)
      for (int64_t g = 0; g < K / G; ++g) {
        if (L->fmt == SVDQ_FMT_INT4_G64) {
          uint16_t s;
          std::memcpy(&s, h.data() + w.sx + 2 * int4_xscale_pos(m, g, K), 2);
          static_cast<uint16_t*>(scales)[size_t(m) * (K / G) + g] = s;
        } else {
          static_cast<uint8_t*>(scales)[size_t(m) * (K / G) + g] = h[w.sx + mx_scale_pos(m, g, K)];
        }
      }
  }
  if (t) {
    const uint16_t* tt = reinterpret_cast<const uint16_t*>(h.data() + w.t);
    uint16_t* o = static_cast<uint16_t*>(t);
    const int ra = L->rank_active;
    for (int64_t m = 0; m < M; ++m)
      for (int j = 0; j < ra; ++j) o[size_t(m) * ra + j] = tt[lr_pos(m, j, L->rank_slots, L->fmt)];
  }
  return SVDQ_OK;
}

extern "C" svdq_status svdq_svd_factors(const void* W_host, int64_t K, int64_t N, int64_t ldw, svdq_dtype dtype,
                                        const float* act_absmax_host, int rank, double* L1, double* L2,
                                        double* sigma, float* lam_out) {
  if (!W_host || K <= 0 || N <= 0 || ldw < N || rank < 0 || rank > std::min(K, N)) return SVDQ_ERR_INVALID_ARG;
  if (dtype != SVDQ_F16 && dtype != SVDQ_BF16) return SVDQ_ERR_INVALID_ARG;
  const uint16_t* Wb = static_cast<const uint16_t*>(W_host);
  std::vector<double> A(size_t(K) * N);
  std::vector<float> lam(K);
  for (int64_t j = 0; j < K; ++j) {
    float w = 0.0f;
    for (int64_t n = 0; n < N; ++n) w = std::fmax(w, std::fabs(h16_to_f32(Wb[j * ldw + n], dtype)));
    float a = act_absmax_host ? act_absmax_host[j] : 0.0f;
    float l = 1.0f;
    if (a > 0.0f && w > 0.0f) {
      float ratio = a / w;
      float sq = std::sqrt(ratio);
      if (std::isfinite(ratio) && ratio > 0.0f && std::isfinite(sq) && sq > 0.0f) l = sq;
    }
    lam[j] = l;
    for (int64_t n = 0; n < N; ++n) A[size_t(j) * N + n] = double(l) * double(h16_to_f32(Wb[j * ldw + n], dtype));
  }
  if (lam_out) std::memcpy(lam_out, lam.data(), size_t(K) * 4);
  if (rank == 0) return SVDQ_OK;
  std::vector<double> l1(size_t(K) * rank), l2(size_t(rank) * N), sg(rank);
  if (!truncated_svd(A.data(), K, N, rank, l1.data(), l2.data(), sg.data())) return SVDQ_ERR_NUMERIC;
  if (L1) std::memcpy(L1, l1.data(), l1.size() * 8);
  if (L2) std::memcpy(L2, l2.data(), l2.size() * 8);
  if (sigma) std::memcpy(sigma, sg.data(), sg.size() * 8);
  return SVDQ_OK;
}
