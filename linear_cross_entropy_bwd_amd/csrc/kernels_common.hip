// Bandwidth-light kernels around the three contractions:
//   label scan (valid-row count), partial-LSE merge and per-row loss,
//   in-place softmax-minus-one-hot gradient, the target-logit pre-pass and the
//   patch of the per-row factor form of that gradient, split-vocabulary dH
//   reduction, and the fixed-order loss reduction.
#include "device_util.h"
#include "flce_internal.h"

#include <math.h>

namespace flce {

namespace {

constexpr int kScanThreads = 1024;

// Number of rows whose label is not ignore_index; also zeroes the per-chunk
// target-logit slots that the logits epilogue fills.
__global__ __launch_bounds__(kScanThreads) void label_scan_kernel(const int64_t* __restrict__ labels, int64_t n,
                                                                  int64_t ignore_index, int32_t* __restrict__ nvalid,
                                                                  float* __restrict__ zy, int64_t chunk) {
  __shared__ int32_t part[kScanThreads / 64];
  int32_t cnt = 0;
  for (int64_t i = threadIdx.x; i < n; i += kScanThreads) cnt += labels[i] != ignore_index ? 1 : 0;
  for (int64_t i = threadIdx.x; i < chunk; i += kScanThreads) zy[i] = 0.0f;
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t t = 0;
    for (int k = 0; k < kScanThreads / 64; ++k) t += part[k];
    *nvalid = t;
  }
}

__device__ __forceinline__ float row_scale(int32_t nvalid, int32_t reduction) {
  if (reduction == FLCE_SUM) return 1.0f;
  return nvalid > 0 ? 1.0f / static_cast<float>(nvalid) : 0.0f;
}

// Merge the per-group (max, sum-exp) partials of each chunk row into
//   lse = m + log(sum_g s_g * exp(m_g - m)),  m = max_g m_g
// (the online log-sum-exp of the blog's section "1. Fused Linear Cross-Entropy
// with Online LogSumExp", step 3, done as an exact two-pass merge), and the
// row's NLL lse - z_y.  With the gradient, each partial max is replaced by
// the factor scale_i * exp(m_g - lse) that turns the stored exp(z - m_g) into
// the scaled softmax, and the value the target column takes is precomputed.
constexpr int kMergeRows = 32;    // 128-byte segments of one group's partials
constexpr int kMergeSlices = 32;

__global__ __launch_bounds__(kMergeRows* kMergeSlices) void lse_merge_kernel(
    float* __restrict__ pm, const float* __restrict__ ps, int64_t C, int64_t G, int64_t rows,
    const int64_t* __restrict__ labels, int64_t ignore_index, int64_t v, const int32_t* __restrict__ nvalid,
    int32_t reduction, float* __restrict__ zy, float* __restrict__ gy, float* __restrict__ lse_rows,
    float* __restrict__ loss_rows, float* __restrict__ zy_rows, int with_grad, const float* __restrict__ uref,
    const int32_t* __restrict__ flag, float* __restrict__ rowf) {
  __shared__ float red[kMergeSlices][kMergeRows];
  __shared__ float row_lse[kMergeRows];
  const int r = threadIdx.x % kMergeRows;
  const int sl = threadIdx.x / kMergeRows;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kMergeRows + r;
  const bool live = t < rows;

  float m = -INFINITY;
  if (live)
#pragma unroll 4
    for (int64_t g = sl; g < G; g += kMergeSlices) m = fmaxf(m, pm[g * C + t]);
  red[sl][r] = m;
  __syncthreads();
  m = red[0][r];
  for (int k = 1; k < kMergeSlices; ++k) m = fmaxf(m, red[k][r]);
  __syncthreads();

  float s = 0.0f;
  if (live)
#pragma unroll 4
    for (int64_t g = sl; g < G; g += kMergeSlices) {
      const float mg = pm[g * C + t];
      s += ps[g * C + t] * fast_exp(mg - m);
    }
  red[sl][r] = s;
  __syncthreads();
  if (sl == 0) {
    float tot = 0.0f;
    for (int k = 0; k < kMergeSlices; ++k) tot += red[k][r];
    const float l = m + logf(tot);
    row_lse[r] = l;
    if (live) {
      const int64_t y = labels[t];
      const bool valid = y != ignore_index;
      const float z = zy[t];
      zy[t] = 0.0f;  // ready for the next chunk
      lse_rows[t] = l;
      loss_rows[t] = valid ? l - z : 0.0f;
      if (zy_rows != nullptr) zy_rows[t] = valid ? z : 0.0f;
      const float sc = valid ? row_scale(*nvalid, reduction) : 0.0f;
      const bool hit = valid && y >= 0 && y < v;
      if (with_grad == 1) {
        gy[t] = hit ? (fast_exp(z - l) - 1.0f) * sc : 0.0f;
      } else if (with_grad == 2) {
        // Folded: G = F_t * P' with one reference per row, the target logit
        // u_t, or the row max m where the row is flagged (its groups are then
        // brought to m by the patch); the target column of P' takes
        // (exp(z - l) - 1) / exp(ref - l).
        const float ref = flag[t] ? m : uref[t];
        rowf[t] = sc > 0.0f ? sc * fast_exp(ref - l) : 0.0f;
        gy[t] = hit ? fast_exp(z - ref) - fast_exp(l - ref) : 0.0f;
      }
    }
  }
  if (!with_grad) return;
  __syncthreads();
  if (!live) return;
  if (with_grad == 2) {
    // a flagged row's group g holds exp(z - r_g), r_g = max(u_t, m_g - margin):
    // its factor to the common reference m is exp(r_g - m)
    if (!flag[t]) return;
    const float u = uref[t];
    for (int64_t g = sl; g < G; g += kMergeSlices) pm[g * C + t] = fast_exp(fmaxf(u, pm[g * C + t] - kFoldMargin) - m);
    return;
  }
  const float l = row_lse[r];
  const int64_t y = labels[t];
  const float sc = y != ignore_index ? row_scale(*nvalid, reduction) : 0.0f;
  for (int64_t g = sl; g < G; g += kMergeSlices) pm[g * C + t] = sc * fast_exp(pm[g * C + t] - l);
}

// G = P * factor(group, row), the target column takes the precomputed value;
// columns in [v, vp) stay 0.  Each thread rewrites 8 consecutive columns
// (one 16-byte vector for bf16, two for fp32); a group holds whole vectors.
template <typename TP>
__device__ __forceinline__ void grad_vec8(TP* p, float f, int64_t c0, int64_t v, int64_t y, float gt);

template <>
__device__ __forceinline__ void grad_vec8<bf16_t>(bf16_t* p, float f, int64_t c0, int64_t v, int64_t y, float gt) {
  uint4 x = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t c = c0 + 2 * k;
    float lo = bf16_to_f32(static_cast<bf16_t>(w[k] & 0xffffu)) * f;
    float hi = bf16_to_f32(static_cast<bf16_t>(w[k] >> 16)) * f;
    if (c == y) lo = gt;
    if (c + 1 == y) hi = gt;
    if (c >= v) lo = 0.0f;
    if (c + 1 >= v) hi = 0.0f;
    w[k] = pack_bf16x2(lo, hi);
  }
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

template <>
__device__ __forceinline__ void grad_vec8<float>(float* p, float f, int64_t c0, int64_t v, int64_t y, float gt) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float4 x = *reinterpret_cast<const float4*>(p + 4 * h);
    float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t c = c0 + 4 * h + k;
      float g = e[k] * f;
      if (c == y) g = gt;
      if (c >= v) g = 0.0f;
      e[k] = g;
    }
    *reinterpret_cast<float4*>(p + 4 * h) = make_float4(e[0], e[1], e[2], e[3]);
  }
}

constexpr int kGradVecs = 4;  // 8-column vectors per thread

template <typename TP>
__global__ __launch_bounds__(256) void grad_kernel(TP* __restrict__ prob, int64_t vp, int64_t v, int64_t group,
                                                   const float* __restrict__ factor, int64_t C,
                                                   const float* __restrict__ gy, const int64_t* __restrict__ labels) {
  const int64_t t = blockIdx.x;
  const int64_t y = labels[t];
  const float gt = gy[t];
  TP* row = prob + t * vp;
#pragma unroll
  for (int q = 0; q < kGradVecs; ++q) {
    const int64_t c0 = ((static_cast<int64_t>(blockIdx.y) * kGradVecs + q) * 256 + threadIdx.x) * 8;
    if (c0 >= vp) return;
    const float f = c0 < v ? factor[(c0 / group) * C + t] : 0.0f;
    grad_vec8<TP>(row + c0, f, c0, v, y, gt);
  }
}

// Folded backward, before the logits: u_t = h_t . w_{y_t} in fp32, the row's
// reference for the stored P (one wave per row); +1e30 for an ignored row
// (its P and factor are then 0) and -1e30 for a label outside [0, v) (every
// group then exceeds it, which flags the row).  Also clears the row flags.
__global__ __launch_bounds__(256) void target_ref_kernel(const bf16_t* __restrict__ h, const bf16_t* __restrict__ w,
                                                         int64_t d, int64_t v, const int64_t* __restrict__ labels,
                                                         int64_t ignore_index, int64_t rows, float* __restrict__ uref,
                                                         int32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= rows) return;  // whole waves
  const int64_t y = labels[t];
  float u;
  if (y == ignore_index) {
    u = 1e30f;
  } else if (y < 0 || y >= v) {
    u = -1e30f;
  } else {
    const uint4* hr = reinterpret_cast<const uint4*>(h + t * d);
    const uint4* wr = reinterpret_cast<const uint4*>(w + y * d);
    float acc = 0.0f;
    for (int64_t k = lane; k < d / 8; k += 64) {
      const uint4 a = hr[k], b = wr[k];
      const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = fmaf(__uint_as_float(av[q] << 16), __uint_as_float(bv[q] << 16), acc);
        acc = fmaf(__uint_as_float(av[q] & 0xffff0000u), __uint_as_float(bv[q] & 0xffff0000u), acc);
      }
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    u = acc;
  }
  if (lane == 0) {
    uref[t] = u;
    flag[t] = 0;
  }
}

// Folded backward, after the merge (one block per chunk row): the token
// operand of dW, H'_t = bf16(F_t h_t); the target column of P' takes its
// value; a flagged row's groups are rescaled to the common reference.
__global__ __launch_bounds__(256) void fold_patch_kernel(const bf16_t* __restrict__ h, bf16_t* __restrict__ hs,
                                                         int64_t d, bf16_t* __restrict__ prob, int64_t vp, int64_t v,
                                                         int64_t group, const float* __restrict__ factor, int64_t C,
                                                         const float* __restrict__ rowf,
                                                         const int32_t* __restrict__ flag,
                                                         const float* __restrict__ gy,
                                                         const int64_t* __restrict__ labels, int64_t ignore_index) {
  const int64_t t = blockIdx.x;
  const float f = rowf[t];
  const uint4* src = reinterpret_cast<const uint4*>(h + t * d);
  uint4* dst = reinterpret_cast<uint4*>(hs + t * d);
  for (int64_t k = threadIdx.x; k < d / 8; k += 256) {
    const uint4 x = src[k];
    const uint32_t xv[4] = {x.x, x.y, x.z, x.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16x2(__uint_as_float(xv[q] << 16) * f, __uint_as_float(xv[q] & 0xffff0000u) * f);
    dst[k] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  const int64_t y = labels[t];
  const bool hit = y != ignore_index && y >= 0 && y < v;
  bf16_t* row = prob + t * vp;
  if (flag[t]) {
    const float gt = gy[t];
    for (int64_t c0 = static_cast<int64_t>(threadIdx.x) * 8; c0 < vp; c0 += 256 * 8) {
      const float fg = c0 < v ? factor[(c0 / group) * C + t] : 0.0f;
      grad_vec8<bf16_t>(row + c0, fg, c0, v, hit ? y : -1, gt);
    }
  } else if (hit && threadIdx.x == 0) {
    row[y] = f32_to_bf16(gy[t]);
  }
}

// x *= *scale in place (fp32 products rounded to the element type), 16-byte
// vectors; a scale of exactly 1 returns at once.
template <typename T>
__global__ __launch_bounds__(256) void scale_kernel(T* __restrict__ x, int64_t count, const float* __restrict__ scale) {
  const float s = *scale;
  if (s == 1.0f) return;
  constexpr int kVec = 16 / sizeof(T);
  const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * kVec;
  if (i0 + kVec <= count) {
    uint4 q = *reinterpret_cast<const uint4*>(x + i0);
    T* e = reinterpret_cast<T*>(&q);
#pragma unroll
    for (int k = 0; k < kVec; ++k) Elem<T>::st(e, k, Elem<T>::ld(e, k) * s);
    *reinterpret_cast<uint4*>(x + i0) = q;
  } else {
    for (int64_t i = i0; i < count; ++i) Elem<T>::st(x, i, Elem<T>::ld(x, i) * s);
  }
}

// dH rows = sum of the split partials (added to what `out` holds when
// accumulating), rounded to the output type.
template <typename TO>
__global__ __launch_bounds__(256) void dh_reduce_kernel(const float* __restrict__ part, int64_t splits,
                                                        int64_t stride, int64_t count, int accumulate,
                                                        TO* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  float acc = accumulate ? Elem<TO>::ld(out, i) : 0.0f;
  for (int64_t s = 0; s < splits; ++s) acc += part[s * stride + i];
  Elem<TO>::st(out, i, acc);
}

// Labels of a vocabulary shard: id - first (wrapping), so that a label in the
// shard becomes its row in the shard's W and every other label falls outside
// [0, v_shard); the ignore value is shifted alike by the caller.
__global__ __launch_bounds__(256) void shift_labels_kernel(const int64_t* __restrict__ labels, int64_t n,
                                                           int64_t first, int64_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) out[i] = static_cast<int64_t>(static_cast<uint64_t>(labels[i]) - static_cast<uint64_t>(first));
}

// Merge the per-shard partials of each row: lse = log sum_p exp(lse_p) (max
// first), the target logit is the one shard's value that holds the label (the
// others hold 0), and the row's NLL lse - z_y.
__global__ __launch_bounds__(256) void shard_merge_kernel(const float* __restrict__ lse_parts,
                                                          const float* __restrict__ zy_parts, int64_t shards,
                                                          int64_t n, const int64_t* __restrict__ labels,
                                                          int64_t ignore_index, float* __restrict__ lse_out,
                                                          float* __restrict__ loss_rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float m = -INFINITY;
  for (int64_t q = 0; q < shards; ++q) m = fmaxf(m, lse_parts[q * n + i]);
  float sum = 0.0f, zy = 0.0f;
  for (int64_t q = 0; q < shards; ++q) {
    sum += m == -INFINITY ? 0.0f : fast_exp(lse_parts[q * n + i] - m);
    zy += zy_parts[q * n + i];
  }
  const float l = m + logf(sum);
  lse_out[i] = l;
  loss_rows[i] = labels[i] != ignore_index ? l - zy : 0.0f;
}

// out[r, k] = bf16(e4m3(q[r, k]) * scale[r]), rounded to nearest even.  e4m3
// (OCP): sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
// subnormal (m / 8 * 2^-6), S.1111.111 is NaN.  Each thread converts 16 bytes.
__global__ __launch_bounds__(256) void dequant_e4m3_kernel(const uint8_t* __restrict__ q,
                                                           const float* __restrict__ scale, int64_t rows,
                                                           int64_t d, bf16_t* __restrict__ out) {
  const int64_t vecs_per_row = d / 16;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * vecs_per_row) return;
  const int64_t r = i / vecs_per_row;
  const float s = scale[r];
  const uint4 u = *reinterpret_cast<const uint4*>(q + i * 16);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float f[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = (w[j >> 1] >> (8 * (2 * (j & 1) + h))) & 0xffu;
      const uint32_t e = (c >> 3) & 0xfu, m = c & 0x7u;
      float v = e == 0 ? static_cast<float>(m) * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
      if (e == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
      f[h] = ((c & 0x80u) ? -v : v) * s;
    }
    o[j] = pack_bf16x2(f[0], f[1]);
  }
  uint4* dst = reinterpret_cast<uint4*>(out + i * 16);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// loss = scale * sum_i loss_rows[i], summed in fp64 in a fixed order.
__global__ __launch_bounds__(1024) void loss_reduce_kernel(const float* __restrict__ loss_rows, int64_t n,
                                                           const int32_t* __restrict__ nvalid, int32_t reduction,
                                                           float* __restrict__ loss_out) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) acc += static_cast<double>(loss_rows[i]);
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int32_t nv = *nvalid;
    const double sc = reduction == FLCE_SUM ? 1.0 : (nv > 0 ? 1.0 / static_cast<double>(nv) : 0.0);
    *loss_out = static_cast<float>(part[0] * sc);
  }
}

}  // namespace

hipError_t launch_label_scan(const Plan& p, const Work& w, const int64_t* labels, int64_t ignore_index,
                             hipStream_t s) {
  label_scan_kernel<<<1, kScanThreads, 0, s>>>(labels, p.n, ignore_index, w.nvalid, w.zy, p.chunk);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const Plan& p, const Work& w, const ChunkArgs& a, int with_grad, hipStream_t s) {
  const int64_t blocks = (a.rows + kMergeRows - 1) / kMergeRows;
  lse_merge_kernel<<<static_cast<unsigned>(blocks), kMergeRows * kMergeSlices, 0, s>>>(
      w.pm, w.ps, p.chunk, p.ngroups, a.rows, a.labels, a.ignore_index, p.v, w.nvalid, a.reduction, w.zy, w.gy,
      a.lse_rows, w.loss_rows + a.row0, a.zy_rows, with_grad, w.uref, w.flag, w.rowf);
  return hipGetLastError();
}

hipError_t launch_target_ref(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((a.rows + 3) / 4);
  target_ref_kernel<<<blocks, 256, 0, s>>>(static_cast<const bf16_t*>(a.h), static_cast<const bf16_t*>(a.w), p.d, p.v,
                                           a.labels, a.ignore_index, a.rows, w.uref, w.flag);
  return hipGetLastError();
}

hipError_t launch_fold_patch(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s) {
  fold_patch_kernel<<<static_cast<unsigned>(a.rows), 256, 0, s>>>(
      static_cast<const bf16_t*>(a.h), static_cast<bf16_t*>(w.hs), p.d, static_cast<bf16_t*>(w.prob), p.vp, p.v,
      p.group, w.pm, p.chunk, w.rowf, w.flag, w.gy, a.labels, a.ignore_index);
  return hipGetLastError();
}

hipError_t launch_grad(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>((p.vp / 8 + 256 * kGradVecs - 1) / (256 * kGradVecs)));
  if (p.engine == ENGINE_MFMA)
    grad_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<bf16_t*>(w.prob), p.vp, p.v, p.group, w.pm, p.chunk, w.gy,
                                             a.labels);
  else
    grad_kernel<float><<<grid, 256, 0, s>>>(static_cast<float*>(w.prob), p.vp, p.v, p.group, w.pm, p.chunk, w.gy,
                                            a.labels);
  return hipGetLastError();
}

hipError_t launch_dh_reduce(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s) {
  const int64_t count = a.rows * p.d;
  const unsigned blocks = static_cast<unsigned>((count + 255) / 256);
  if (p.dtype == FLCE_BF16 && !a.dh_f32)
    dh_reduce_kernel<bf16_t><<<blocks, 256, 0, s>>>(w.dhpart, p.dh_splits, p.chunk * p.d, count, 0,
                                                    static_cast<bf16_t*>(a.dh));
  else
    dh_reduce_kernel<float><<<blocks, 256, 0, s>>>(w.dhpart, p.dh_splits, p.chunk * p.d, count, a.dh_accumulate,
                                                   static_cast<float*>(a.dh));
  return hipGetLastError();
}

hipError_t launch_loss_reduce(const Plan& p, const Work& w, int32_t reduction, float* loss_out, hipStream_t s) {
  loss_reduce_kernel<<<1, 1024, 0, s>>>(w.loss_rows, p.n, w.nvalid, reduction, loss_out);
  return hipGetLastError();
}

}  // namespace flce

namespace flce {

hipError_t launch_label_count(const int64_t* labels, int64_t n, int64_t ignore_index, int32_t* nvalid, hipStream_t s) {
  label_scan_kernel<<<1, kScanThreads, 0, s>>>(labels, n, ignore_index, nvalid, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_loss_sum(const float* loss_rows, int64_t n, const int32_t* nvalid, int32_t reduction,
                           float* loss_out, hipStream_t s) {
  loss_reduce_kernel<<<1, 1024, 0, s>>>(loss_rows, n, nvalid, reduction, loss_out);
  return hipGetLastError();
}

hipError_t launch_shift_labels(const int64_t* labels, int64_t n, int64_t first, int64_t* out, hipStream_t s) {
  shift_labels_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(labels, n, first, out);
  return hipGetLastError();
}

hipError_t launch_shard_merge(const float* lse_parts, const float* zy_parts, int64_t shards, int64_t n,
                              const int64_t* labels, int64_t ignore_index, float* lse_out, float* loss_rows,
                              hipStream_t s) {
  shard_merge_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(lse_parts, zy_parts, shards, n, labels,
                                                                             ignore_index, lse_out, loss_rows);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* parts, int64_t num_parts, int64_t count, int32_t dtype, void* out,
                            hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((count + 255) / 256);
  if (dtype == FLCE_BF16)
    dh_reduce_kernel<bf16_t><<<blocks, 256, 0, s>>>(parts, num_parts, count, count, 0, static_cast<bf16_t*>(out));
  else
    dh_reduce_kernel<float><<<blocks, 256, 0, s>>>(parts, num_parts, count, count, 0, static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_scale(void* x, int64_t count, int32_t dtype, const float* scale, hipStream_t s) {
  const int64_t vec = dtype == FLCE_BF16 ? 8 : 4;
  const unsigned blocks = static_cast<unsigned>((count + 256 * vec - 1) / (256 * vec));
  if (dtype == FLCE_BF16)
    scale_kernel<bf16_t><<<blocks, 256, 0, s>>>(static_cast<bf16_t*>(x), count, scale);
  else
    scale_kernel<float><<<blocks, 256, 0, s>>>(static_cast<float*>(x), count, scale);
  return hipGetLastError();
}

hipError_t launch_dequant_e4m3(const void* q, const float* scale, int64_t rows, int64_t d, void* out, hipStream_t s) {
  const int64_t n = rows * (d / 16);
  dequant_e4m3_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      static_cast<const uint8_t*>(q), scale, rows, d, static_cast<bf16_t*>(out));
  return hipGetLastError();
}

}  // namespace flce
