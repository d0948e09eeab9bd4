// dkv_layout.hip -- moving per-token rows between the two packings of a micro-batch
// ("DualKV", arXiv 2605.15422, §2.1 eq. (1), §2.2 eq. (5), §2.3, App. A.2 / A.5).
//
// The N-copy packing stores, for every response i, its prompt's rows followed by its
// own rows; the single-prompt packing stores each prompt once (all prompts first,
// then all responses).  Every per-token operation of the model can run on the smaller
// packing; these kernels convert activations and gradients between the two and
// provide the first-token predictor rows (the last prompt token's hidden state
// predicts the first token of every response of its prompt, §2.3).
//
// One kernel serves all of them: a work item names up to 16 consecutive rows, each the
// sum of the same-offset rows of `nsrc` input row ranges (fp32 accumulation, rounded
// once), a plain copy when nsrc == 1 and zeros when nsrc == 0, written to `ndst` output
// ranges (a prompt chunk is read once and written to every copy of its group).  Rows move in
// 16-byte vectors, consecutive threads on consecutive vectors (coalesced); the work is
// HBM-bound.
#include "dkv_device.h"
#include "dkv_launch.h"

namespace dkv {

template <typename T>
__global__ __launch_bounds__(256) void row_sum_kernel(const T *__restrict__ in, T *__restrict__ out,
                                                      const RowItem *__restrict__ items,
                                                      const int32_t *__restrict__ tab,
                                                      int row_vecs) {
  constexpr int E = 16 / sizeof(T);            // elements per 16-byte vector
  constexpr int U = 4;                         // vectors in flight per thread
  const RowItem it = items[blockIdx.x];
  const int32_t *src = tab + it.tab_off, *dst = src + it.nsrc;
  const int nv = it.nrows * row_vecs;
  const long row_elems = (long)row_vecs * E;
  if (it.nsrc == 1) {   // a copy: U loads issued before their stores to every destination
    // the item's rows are consecutive in every range: one run of nv vectors each
    const uint4 *s0 = reinterpret_cast<const uint4 *>(in + (long)src[0] * row_elems);
    int idx = threadIdx.x;
    for (; idx + (U - 1) * 256 < nv; idx += U * 256) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = s0[idx + u * 256];
      for (int k = 0; k < it.ndst; ++k) {
        uint4 *d0 = reinterpret_cast<uint4 *>(out + (long)dst[k] * row_elems);
#pragma unroll
        for (int u = 0; u < U; ++u) d0[idx + u * 256] = v[u];
      }
    }
    for (; idx < nv; idx += 256) {
      const uint4 v = s0[idx];
      for (int k = 0; k < it.ndst; ++k) reinterpret_cast<uint4 *>(out + (long)dst[k] * row_elems)[idx] = v;
    }
    return;
  }
  for (int idx = threadIdx.x; idx < nv; idx += 256) {
    const int r = idx / row_vecs, c = idx - r * row_vecs;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    int s = 0;
    for (; s + 1 < it.nsrc; s += 2) {   // two source rows in flight
      const uint4 v0 = *(reinterpret_cast<const uint4 *>(in + (long)(src[s] + r) * row_elems) + c);
      const uint4 v1 = *(reinterpret_cast<const uint4 *>(in + (long)(src[s + 1] + r) * row_elems) + c);
      const T *x0 = reinterpret_cast<const T *>(&v0);
      const T *x1 = reinterpret_cast<const T *>(&v1);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = (acc[e] + to_f32(x0[e])) + to_f32(x1[e]);
    }
    if (s < it.nsrc) {
      const uint4 v = *(reinterpret_cast<const uint4 *>(in + (long)(src[s] + r) * row_elems) + c);
      const T *x = reinterpret_cast<const T *>(&v);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += to_f32(x[e]);
    }
    uint4 o;
    T *y = reinterpret_cast<T *>(&o);
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = from_f32<T>(acc[e]);
    for (int k = 0; k < it.ndst; ++k)
      *(reinterpret_cast<uint4 *>(out + (long)(dst[k] + r) * row_elems) + c) = o;
  }
}

hipError_t launch_row_sum(int dtype, const void *in, void *out, const RowItem *items, int n_items,
                          const int32_t *tab, int row_vecs, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (dtype == 2)
    hipLaunchKernelGGL(row_sum_kernel<f16>, dim3(n_items), dim3(256), 0, s,
                       reinterpret_cast<const f16 *>(in), reinterpret_cast<f16 *>(out), items,
                       tab, row_vecs);
  else if (dtype == 0)
    hipLaunchKernelGGL(row_sum_kernel<h16>, dim3(n_items), dim3(256), 0, s,
                       reinterpret_cast<const h16 *>(in), reinterpret_cast<h16 *>(out), items,
                       tab, row_vecs);
  else
    hipLaunchKernelGGL(row_sum_kernel<float>, dim3(n_items), dim3(256), 0, s,
                       reinterpret_cast<const float *>(in), reinterpret_cast<float *>(out), items,
                       tab, row_vecs);
  return hipGetLastError();
}

}  // namespace dkv
