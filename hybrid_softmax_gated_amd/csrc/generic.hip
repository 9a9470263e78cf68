// Plain VALU kernels for the shapes the MFMA kernels do not take (float32
// io, or head dimension 16): the small exactness workloads. Same method and
// same data layout as the MFMA path ("Technical Summary: Attend Locally,
// Remember Linearly (ARL2)", sections 2.1 and 2.2), fp32 arithmetic
// throughout, one thread per query (attention and read) or per output
// element (state update).
#include "arl2_device.h"
#include "arl2_kernels.h"

#include <math.h>

namespace arl2 {
namespace {

__device__ __forceinline__ float ld(const float *p) { return *p; }
__device__ __forceinline__ float ld(const bf16 *p) { return (float)*p; }
__device__ __forceinline__ void st(float *p, float x) { *p = x; }
__device__ __forceinline__ void st(bf16 *p, float x) { *p = (bf16)x; }

// O_intra[b][h][q][:] = softmax(q k^T / sqrt(d)) v for one query per thread.
template <typename T, int Dm>
__global__ __launch_bounds__(64) void gen_attn_kernel(const T *q, const T *k, const T *v, int H,
                                                      int Lq, int Lk, float *o_intra) {
  const int qi = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (qi >= Lq) return;
  const float scale = 1.f / sqrtf((float)Dm);
  const T *qp = q + (((int64_t)b * Lq + qi) * H + h) * Dm;
  float qv[Dm], o[Dm];
#pragma unroll
  for (int e = 0; e < Dm; ++e) {
    qv[e] = ld(qp + e);
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < Lk; ++j) {
    const T *kp = k + (((int64_t)b * Lk + j) * H + h) * Dm;
    const T *vp = v + (((int64_t)b * Lk + j) * H + h) * Dm;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < Dm; ++e) s = fmaf(qv[e], ld(kp + e), s);
    s *= scale;
    if (s > m) {
      const float r = expf(m - s);
      l *= r;
#pragma unroll
      for (int e = 0; e < Dm; ++e) o[e] *= r;
      m = s;
    }
    const float pj = expf(s - m);
    l += pj;
#pragma unroll
    for (int e = 0; e < Dm; ++e) o[e] = fmaf(pj, ld(vp + e), o[e]);
  }
  float *op = o_intra + (((int64_t)b * H + h) * Lq + qi) * Dm;
  const float il = 1.f / l;
#pragma unroll
  for (int e = 0; e < Dm; ++e) op[e] = o[e] * il;
}

// out = O_intra + L2norm(q W_q) S (or O_intra alone), one query per thread.
template <typename T, int Dm>
__global__ __launch_bounds__(64) void gen_inter_combine_kernel(const T *q, const T *Wq,
                                                               const float *S, const float *o_intra,
                                                               int H, int L, T *out,
                                                               int with_inter) {
  const int qi = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (qi >= L) return;
  const float *oi = o_intra + (((int64_t)b * H + h) * L + qi) * Dm;
  T *op = out + (((int64_t)b * L + qi) * H + h) * Dm;
  if (!with_inter) {
    for (int e = 0; e < Dm; ++e) st(op + e, oi[e]);
    return;
  }
  const T *qp = q + (((int64_t)b * L + qi) * H + h) * Dm;
  const T *W = Wq + (int64_t)h * Dm * Dm;
  const float *Sh = S + ((int64_t)b * H + h) * Dm * Dm;
  float qw[Dm];
#pragma unroll
  for (int e = 0; e < Dm; ++e) qw[e] = 0.f;
  for (int i = 0; i < Dm; ++i) {
    const float x = ld(qp + i);
#pragma unroll
    for (int e = 0; e < Dm; ++e) qw[e] = fmaf(x, ld(W + i * Dm + e), qw[e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < Dm; ++e) ss = fmaf(qw[e], qw[e], ss);
  const float inv = 1.f / fmaxf(sqrtf(ss), kL2Eps);
  for (int e = 0; e < Dm; ++e) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < Dm; ++i) acc = fmaf(qw[i] * inv, Sh[i * Dm + e], acc);
    st(op + e, oi[e] + acc);
  }
}

// dS_c = K'^T diag(beta) (V' - K' S) over one chunk of kGenChunk tokens.
template <typename T, int Dm>
__global__ __launch_bounds__(256) void gen_delta_partial_kernel(const T *k, const T *v,
                                                                const T *Wk, const T *Wv,
                                                                const float *S, const float *beta,
                                                                int H, int L, int nchunk,
                                                                float *ws_dS) {
  constexpr int C = kGenChunk;
  __shared__ float Kp[C * Dm];
  __shared__ float Rb[C * Dm];
  __shared__ float inv[C];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tbase = chunk * C;
  const T *Wkh = Wk + (int64_t)h * Dm * Dm;
  const T *Wvh = Wv + (int64_t)h * Dm * Dm;
  const float *Sh = S + ((int64_t)b * H + h) * Dm * Dm;

  for (int idx = tid; idx < C * Dm; idx += 256) {
    const int tt = idx / Dm, e = idx % Dm, t = tbase + tt;
    float ka = 0.f, va = 0.f;
    if (t < L) {
      const int64_t row = (((int64_t)b * L + t) * H + h) * Dm;
      for (int i = 0; i < Dm; ++i) {
        ka = fmaf(ld(k + row + i), ld(Wkh + i * Dm + e), ka);
        va = fmaf(ld(v + row + i), ld(Wvh + i * Dm + e), va);
      }
    }
    Kp[idx] = ka;
    Rb[idx] = va;
  }
  __syncthreads();
  if (tid < C) {
    float ss = 0.f;
    for (int e = 0; e < Dm; ++e) ss = fmaf(Kp[tid * Dm + e], Kp[tid * Dm + e], ss);
    inv[tid] = 1.f / fmaxf(sqrtf(ss), kL2Eps);
  }
  __syncthreads();
  for (int idx = tid; idx < C * Dm; idx += 256) Kp[idx] *= inv[idx / Dm];
  __syncthreads();
  for (int idx = tid; idx < C * Dm; idx += 256) {
    const int tt = idx / Dm, e = idx % Dm, t = tbase + tt;
    float ks = 0.f;
    for (int i = 0; i < Dm; ++i) ks = fmaf(Kp[tt * Dm + i], Sh[i * Dm + e], ks);
    const float bt = t < L ? beta[((int64_t)b * L + t) * H + h] : 0.f;
    Rb[idx] = (Rb[idx] - ks) * bt;
  }
  __syncthreads();
  float *wd = ws_dS + (((int64_t)b * H + h) * nchunk + chunk) * Dm * Dm;
  for (int idx = tid; idx < Dm * Dm; idx += 256) {
    const int i = idx / Dm, e = idx % Dm;
    float acc = 0.f;
    for (int tt = 0; tt < C; ++tt) acc = fmaf(Kp[tt * Dm + i], Rb[tt * Dm + e], acc);
    wd[idx] = acc;
  }
}

template <typename T, int Dm>
hipError_t gen_attention(const void *q, const void *k, const void *v, int B, int H, int Lq, int Lk,
                         float *o_intra, hipStream_t s) {
  dim3 grid((unsigned)((Lq + 63) / 64), (unsigned)H, (unsigned)B);
  launch((gen_attn_kernel<T, Dm>), grid, dim3(64), 0, s, (const T *)q, (const T *)k,
                     (const T *)v, H, Lq, Lk, o_intra);
  return hipGetLastError();
}

template <typename T, int Dm>
hipError_t gen_inter_combine(const void *q, const void *Wq, const float *S, const float *o_intra,
                             int B, int H, int L, void *out, bool with_inter, hipStream_t s) {
  dim3 grid((unsigned)((L + 63) / 64), (unsigned)H, (unsigned)B);
  launch((gen_inter_combine_kernel<T, Dm>), grid, dim3(64), 0, s, (const T *)q,
                     (const T *)Wq, S, o_intra, H, L, (T *)out, with_inter ? 1 : 0);
  return hipGetLastError();
}

template <typename T, int Dm>
hipError_t gen_delta_partial(const void *k, const void *v, const void *Wk, const void *Wv,
                             const float *S, const float *beta, int B, int H, int L, float *ws_dS,
                             hipStream_t s) {
  const int nchunk = (L + kGenChunk - 1) / kGenChunk;
  dim3 grid((unsigned)nchunk, (unsigned)H, (unsigned)B);
  launch((gen_delta_partial_kernel<T, Dm>), grid, dim3(256), 0, s, (const T *)k,
                     (const T *)v, (const T *)Wk, (const T *)Wv, S, beta, H, L, nchunk, ws_dS);
  return hipGetLastError();
}

}  // namespace

#define ARL2_GEN_DISPATCH(FN, ...)                                   \
  do {                                                               \
    if (dtype == 1 && d == 16) return FN<float, 16>(__VA_ARGS__);    \
    if (dtype == 1 && d == 128) return FN<float, 128>(__VA_ARGS__);  \
    if (dtype == 0 && d == 16) return FN<bf16, 16>(__VA_ARGS__);     \
    if (dtype == 0 && d == 128) return FN<bf16, 128>(__VA_ARGS__);   \
    return hipErrorInvalidValue;                                     \
  } while (0)

hipError_t launch_generic_attention(int dtype, int d, const void *q, const void *k, const void *v,
                                    int B, int H, int Lq, int Lk, float *o_intra, hipStream_t s) {
  ARL2_GEN_DISPATCH(gen_attention, q, k, v, B, H, Lq, Lk, o_intra, s);
}

hipError_t launch_generic_inter_combine(int dtype, int d, const void *q, const void *Wq,
                                        const float *S, const float *o_intra, int B, int H, int L,
                                        void *out, bool with_inter, hipStream_t s) {
  ARL2_GEN_DISPATCH(gen_inter_combine, q, Wq, S, o_intra, B, H, L, out, with_inter, s);
}

hipError_t launch_generic_delta_partial(int dtype, int d, const void *k, const void *v,
                                        const void *Wk, const void *Wv, const float *S,
                                        const float *beta, int B, int H, int L, float *ws_dS,
                                        hipStream_t s) {
  ARL2_GEN_DISPATCH(gen_delta_partial, k, v, Wk, Wv, S, beta, B, H, L, ws_dS, s);
}

}  // namespace arl2
