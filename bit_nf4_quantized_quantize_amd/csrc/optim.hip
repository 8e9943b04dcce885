// The LoRA-only optimizer step for gfx950: global gradient-norm clipping and
// AdamW over one flat buffer of LoRA parameters.
//
// QLoRA (Dettmers et al., arXiv 2305.14314): section 3 "Paged Optimizers"
// (optimizer states that live in memory the CPU can hold and that are paged
// to the GPU for the update step) and Appendix B.2 "Hyperparameters" (Adam
// beta2 0.999, maximum gradient norm 0.3, constant learning rate); only the
// adapters are trained (section 3 "QLoRA", after Eq. 6).  Read as AdamW with
// decoupled weight decay and clip scale min(1, max_norm / (||g|| + 1e-6)).
//
// Both kernels are streams over the parameters (HBM-bound; 28 bytes per
// parameter for the step with a bf16 copy of the updated weights).  The
// states may live in pinned host memory, which the step kernel reads and
// writes in place over the host link.
#include "device.h"
#include "launch.h"

namespace qlora {

constexpr int OPT_T = kOptThreads;

// Sum of squares of grad[0, n) (bf16), one fp64 partial per workgroup,
// accumulated in a fixed order: thread t takes elements 4(t + k T) .. +3 of
// its workgroup's grid-stride sweep, then the wave and workgroup sums are
// formed by a fixed butterfly and a fixed sum over waves.
__global__ __launch_bounds__(OPT_T) void grad_sqnorm_kernel(const uint16_t* __restrict__ g, int64_t n,
                                                            double* __restrict__ partials) {
  __shared__ double s_w[OPT_T / 64];
  const int64_t stride = (int64_t)gridDim.x * OPT_T * 4;
  double acc = 0.0;
  for (int64_t i = ((int64_t)blockIdx.x * OPT_T + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 3 < n) {
      const uint2 v = *reinterpret_cast<const uint2*>(g + i);
      const float a = __uint_as_float(v.x << 16), b = __uint_as_float(v.x & 0xFFFF0000u);
      const float c = __uint_as_float(v.y << 16), d = __uint_as_float(v.y & 0xFFFF0000u);
      acc += (double)a * a + (double)b * b + (double)c * c + (double)d * d;
    } else {
      for (int64_t j = i; j < n; ++j) {
        const float a = bf2f(g[j]);
        acc += (double)a * a;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < OPT_T / 64; ++w) t += s_w[w];
    partials[blockIdx.x] = t;
  }
}

// scale = min(1, max_norm / (sqrt(sum of partials) + 1e-6)).  One wave: lane
// l adds partials l, l + 64, ... in order (all loads in flight together),
// then a fixed butterfly adds the lanes.
__global__ __launch_bounds__(64) void clip_finish_kernel(const double* __restrict__ partials, int parts,
                                                         float max_norm, float* __restrict__ scale) {
  static_assert(kOptMaxParts % 64 == 0, "partials per lane");
  double v[kOptMaxParts / 64];
#pragma unroll
  for (int k = 0; k < kOptMaxParts / 64; ++k) {
    const int i = (int)threadIdx.x + 64 * k;
    v[k] = i < parts ? partials[i] : 0.0;
  }
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < kOptMaxParts / 64; ++k) t += v[k];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
  if (threadIdx.x == 0) {
    const double c = (double)max_norm / (sqrt(t) + 1e-6);
    *scale = (float)(c < 1.0 ? c : 1.0);
  }
}


hipError_t launch_clip_scale(const uint16_t* g, int64_t n, float max_norm, float* scale, double* partials,
                             hipStream_t stream) {
  const int parts = clip_parts(n);
  hipLaunchKernelGGL(grad_sqnorm_kernel, dim3((unsigned)parts), dim3(OPT_T), 0, stream, g, n, partials);
  hipLaunchKernelGGL(clip_finish_kernel, dim3(1), dim3(64), 0, stream, partials, parts, max_norm, scale);
  return hipGetLastError();
}

struct AdamWArgs {
  float lr, beta1, beta2, eps, decay;  // decay = 1 - lr * weight_decay
  float inv_bc1, inv_sqrt_bc2;         // 1 / (1 - beta1^t), 1 / sqrt(1 - beta2^t)
};

__device__ __forceinline__ float adamw_one(float p, float g, float& m, float& v, const AdamWArgs& a) {
  m = a.beta1 * m + (1.0f - a.beta1) * g;
  v = a.beta2 * v + (1.0f - a.beta2) * (g * g);
  const float denom = sqrtf(v) * a.inv_sqrt_bc2 + a.eps;
  return p * a.decay - (a.lr * a.inv_bc1) * (m / denom);
}

// One AdamW step over n parameters, 4 per thread and iteration.
__global__ __launch_bounds__(OPT_T) void adamw_kernel(float* __restrict__ p, uint16_t* __restrict__ p_bf16,
                                                      const uint16_t* __restrict__ g, float* __restrict__ m,
                                                      float* __restrict__ v, int64_t n,
                                                      const float* __restrict__ gscale, AdamWArgs a) {
  const float sc = gscale ? *gscale : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * OPT_T * 4;
  for (int64_t i = ((int64_t)blockIdx.x * OPT_T + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 3 < n) {
      float4 pv = *reinterpret_cast<const float4*>(p + i);
      float4 mv = *reinterpret_cast<const float4*>(m + i);
      float4 vv = *reinterpret_cast<const float4*>(v + i);
      const uint2 gv = *reinterpret_cast<const uint2*>(g + i);
      pv.x = adamw_one(pv.x, __uint_as_float(gv.x << 16) * sc, mv.x, vv.x, a);
      pv.y = adamw_one(pv.y, __uint_as_float(gv.x & 0xFFFF0000u) * sc, mv.y, vv.y, a);
      pv.z = adamw_one(pv.z, __uint_as_float(gv.y << 16) * sc, mv.z, vv.z, a);
      pv.w = adamw_one(pv.w, __uint_as_float(gv.y & 0xFFFF0000u) * sc, mv.w, vv.w, a);
      *reinterpret_cast<float4*>(p + i) = pv;
      *reinterpret_cast<float4*>(m + i) = mv;
      *reinterpret_cast<float4*>(v + i) = vv;
      if (p_bf16) *reinterpret_cast<uint2*>(p_bf16 + i) = make_uint2(pack_bf2(pv.x, pv.y), pack_bf2(pv.z, pv.w));
    } else {
      for (int64_t j = i; j < n; ++j) {
        float mj = m[j], vj = v[j];
        const float pj = adamw_one(p[j], bf2f(g[j]) * sc, mj, vj, a);
        p[j] = pj;
        m[j] = mj;
        v[j] = vj;
        if (p_bf16) p_bf16[j] = f2bf(pj);
      }
    }
  }
}

hipError_t launch_adamw(float* p, uint16_t* p_bf16, const uint16_t* g, float* m, float* v, int64_t n,
                        const float* gscale, float lr, float beta1, float beta2, float eps, float weight_decay,
                        int step, hipStream_t stream) {
  AdamWArgs a;
  a.lr = lr;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.decay = (float)(1.0 - (double)lr * weight_decay);
  a.inv_bc1 = (float)(1.0 / (1.0 - pow((double)beta1, step)));
  a.inv_sqrt_bc2 = (float)(1.0 / sqrt(1.0 - pow((double)beta2, step)));
  const int64_t wgs = (n + OPT_T * 4 - 1) / (OPT_T * 4);
  const unsigned grid = (unsigned)(wgs < 1 ? 1 : (wgs > 2048 ? 2048 : wgs));
  hipLaunchKernelGGL(adamw_kernel, dim3(grid), dim3(OPT_T), 0, stream, p, p_bf16, g, m, v, n, gscale, a);
  return hipGetLastError();
}

// The paged step: the states live in pinned host memory and are paged
// through the device staging area [2 slots][m, v][chunk] floats, chunk by
// chunk.  Slot c % 2 takes chunk c: its states are copied in (host to
// device), updated by the same AdamW kernel as device-resident states, and
// copied back; chunk c + 2 is copied into the slot after chunk c's copy
// back.  With a separate copy stream the copies run on it, ordered against
// the updates by events, so the copies of one chunk overlap the update of
// the other; without one everything runs in order on `stream`.  Either way
// `stream` reaches its end only after the last copy back.
hipError_t launch_adamw_paged(float* p, uint16_t* p_bf16, const uint16_t* g, float* m_host, float* v_host, int64_t n,
                              const float* gscale, float lr, float beta1, float beta2, float eps, float weight_decay,
                              int step, float* staging, int64_t chunk, hipStream_t stream, hipStream_t copy) {
  if (n <= 0) return hipSuccess;
  if (chunk <= 0 || chunk % 256) return hipErrorInvalidValue;
  const int64_t nch = (n + chunk - 1) / chunk;
  const bool two = copy != nullptr && copy != stream;
  hipStream_t cs = two ? copy : stream;
  hipEvent_t ev[6] = {};  // start, end, loaded[2], updated[2]
  hipError_t e = hipSuccess;
  if (two) {
    for (int i = 0; i < 6 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
  }
  auto slot_m = [&](int64_t c) { return staging + ((c & 1) * 2 + 0) * chunk; };
  auto slot_v = [&](int64_t c) { return staging + ((c & 1) * 2 + 1) * chunk; };
  auto len_of = [&](int64_t c) { return (c + 1) * chunk <= n ? chunk : n - c * chunk; };
  auto page_in = [&](int64_t c) {
    const int64_t off = c * chunk, len = len_of(c);
    if (e == hipSuccess) e = hipMemcpyAsync(slot_m(c), m_host + off, len * 4, hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipMemcpyAsync(slot_v(c), v_host + off, len * 4, hipMemcpyHostToDevice, cs);
    if (two && e == hipSuccess) e = hipEventRecord(ev[2 + (c & 1)], cs);
  };
  if (two && e == hipSuccess) e = hipEventRecord(ev[0], stream);  // after the work before this call
  if (two && e == hipSuccess) e = hipStreamWaitEvent(cs, ev[0], 0);
  page_in(0);
  if (nch > 1) page_in(1);
  for (int64_t c = 0; c < nch && e == hipSuccess; ++c) {
    const int64_t off = c * chunk, len = len_of(c);
    if (two) e = hipStreamWaitEvent(stream, ev[2 + (c & 1)], 0);
    if (e == hipSuccess)
      e = launch_adamw(p + off, p_bf16 ? p_bf16 + off : nullptr, g + off, slot_m(c), slot_v(c), len, gscale, lr,
                       beta1, beta2, eps, weight_decay, step, stream);
    if (two && e == hipSuccess) e = hipEventRecord(ev[4 + (c & 1)], stream);
    if (two && e == hipSuccess) e = hipStreamWaitEvent(cs, ev[4 + (c & 1)], 0);
    if (e == hipSuccess) e = hipMemcpyAsync(m_host + off, slot_m(c), len * 4, hipMemcpyDeviceToHost, cs);
    if (e == hipSuccess) e = hipMemcpyAsync(v_host + off, slot_v(c), len * 4, hipMemcpyDeviceToHost, cs);
    if (c + 2 < nch) page_in(c + 2);
  }
  if (two && e == hipSuccess) e = hipEventRecord(ev[1], cs);
  if (two && e == hipSuccess) e = hipStreamWaitEvent(stream, ev[1], 0);
  for (int i = 0; i < 6; ++i)
    if (ev[i]) (void)hipEventDestroy(ev[i]);  // released once the streams have passed them
  return e;
}

}  // namespace qlora
