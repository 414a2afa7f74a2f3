// Layer-level velocity-distillation loss and its gradient (gist.science,
// section 2B): loss = mean of (o_student - o_teacher)^2 over all elements,
// dout = 2 (o_student - o_teacher) / numel.  An HBM stream: each workgroup
// owns one contiguous chunk, writes dout and its fp64 sum of squares; one
// workgroup then adds the chunk sums in chunk order.
#include "sa2_common.h"

namespace sa2 {

constexpr int kDistillGroups = 1024;
constexpr int kDistillThreads = 256;

template <typename T>
__global__ __launch_bounds__(kDistillThreads)
void distill_chunks_kernel(const T* __restrict__ os, const T* __restrict__ ot, size_t n8,
                           double inv_numel, T* __restrict__ dout, double* __restrict__ part) {
  __shared__ double red[kDistillThreads / 64];
  const size_t per = (n8 + gridDim.x - 1) / gridDim.x;        // 8-element units per chunk
  const size_t lo = (size_t)blockIdx.x * per, hi = lo + per < n8 ? lo + per : n8;
  const float g = (float)(2.0 * inv_numel);
  double acc = 0.0;
  for (size_t u = lo + threadIdx.x; u < hi; u += kDistillThreads) {
    float a[8], b[8];
    load8_f32(os + 8 * u, a);
    load8_f32(ot + 8 * u, b);
    float dd[8];
    double sq = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dd[i] = a[i] - b[i];
      sq += (double)dd[i] * (double)dd[i];
    }
    acc += sq;
    store4(dout + 8 * u, dd[0] * g, dd[1] * g, dd[2] * g, dd[3] * g);
    store4(dout + 8 * u + 4, dd[4] * g, dd[5] * g, dd[6] * g, dd[7] * g);
  }
  // fixed-order workgroup sum: lanes by shuffle tree, waves in order
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kDistillThreads / 64; ++w) t += red[w];
    part[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(64)
void distill_total_kernel(const double* __restrict__ part, int n, double inv_numel,
                          double* __restrict__ loss) {
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < n; ++i) t += part[i];
    loss[0] = t * inv_numel;
  }
}

}  // namespace sa2

extern "C" size_t sa2_distill_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  return (size_t)sa2::kDistillGroups * sizeof(double);
}

extern "C" sa2_status sa2_distill_loss_grad(const void* o_student, const void* o_teacher,
                                            int dtype, int B, int H, int N, int d, void* dout,
                                            double* loss, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  using namespace sa2;
  const char* fn = "sa2_distill_loss_grad";
  if (!o_student || !o_teacher || !dout || !loss || !workspace)
    return fail(SA2_EINVAL, std::string(fn) + ": null pointer");
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
    return fail(SA2_EINVAL, std::string(fn) + ": B, H, N, d must be positive");
  if (dtype != SA2_BF16 && dtype != SA2_F32) return fail(SA2_EINVAL, std::string(fn) + ": unknown dtype");
  if (d % 8 != 0) return fail(SA2_EUNSUPPORTED, std::string(fn) + ": d must be a multiple of 8");
  if (!aligned16(o_student) || !aligned16(o_teacher) || !aligned16(dout))
    return fail(SA2_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SA2_EINVAL, std::string(fn) + ": workspace not 256-byte aligned");
  if (workspace_bytes < sa2_distill_workspace_bytes(B, H, N, d))
    return fail(SA2_EINVAL, std::string(fn) + ": workspace smaller than sa2_distill_workspace_bytes()");
  const size_t numel = (size_t)B * H * N * d;
  const double inv = 1.0 / (double)numel;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  double* part = static_cast<double*>(workspace);
  if (dtype == SA2_BF16)
    distill_chunks_kernel<bf16_t><<<kDistillGroups, kDistillThreads, 0, s>>>(
        static_cast<const bf16_t*>(o_student), static_cast<const bf16_t*>(o_teacher), numel / 8,
        inv, static_cast<bf16_t*>(dout), part);
  else
    distill_chunks_kernel<float><<<kDistillGroups, kDistillThreads, 0, s>>>(
        static_cast<const float*>(o_student), static_cast<const float*>(o_teacher), numel / 8,
        inv, static_cast<float*>(dout), part);
  if (sa2_status st = check_launch("distill_chunks_kernel")) return st;
  distill_total_kernel<<<1, 64, 0, s>>>(part, kDistillGroups, inv, loss);
  return check_launch("distill_total_kernel");
}
