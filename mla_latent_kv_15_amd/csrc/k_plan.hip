// Split-KV work plan: the kernels that build it (plan_device.h) and its
// host-side sizes and layout.
#include "plan_device.h"

namespace mla {

namespace {

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanJob job) { plan_build(job); }

// splitk reduction (one output element per thread) and, in work-group 0,
// the plan
__global__ __launch_bounds__(kPlanThreads) void reduce_plan_kernel(int M, int N, int S,
                                                                   const float* __restrict__ part,
                                                                   long split_stride,
                                                                   __bf16* __restrict__ out,
                                                                   long ldo, int blocked,
                                                                   PlanJob job) {
  // the plan in the first work-group (dispatched first), the reduction in the rest
  if (blockIdx.x == 0) {
    plan_build(job);
    return;
  }
  const long idx = (long)(blockIdx.x - 1) * blockDim.x + threadIdx.x;
  if (idx >= (long)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[s * split_stride + (long)m * N + n];
  out[blocked ? blk_index(m, n, N) : (long)m * ldo + n] = (__bf16)v;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int auto_wg_budget() {
  static int cached = 0;
  if (cached > 0) return cached;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0) {
    cached = cus;
  } else {
    (void)hipGetLastError();
    return 256;
  }
  return cached;
}

PlanDims plan_dims(int B, int num_splits) {
  PlanDims d;
  if (num_splits > 0) {
    d.max_segs = B * num_splits;
    d.max_wg = B * num_splits;
  } else {
    d.max_wg = auto_wg_budget();
    d.max_segs = d.max_wg + B;
  }
  return d;
}

size_t plan_bytes(int B, int num_splits) {
  PlanDims d = plan_dims(B, num_splits);
  return align256(sizeof(Seg) * (size_t)d.max_segs) + align256(sizeof(int) * (size_t)B) * 2 +
         align256(sizeof(int) * (size_t)(d.max_wg + 1)) + 256;
}

void carve_plan(void* base, int B, int num_splits, PlanPtrs* p) {
  PlanDims d = plan_dims(B, num_splits);
  char* c = (char*)base;
  p->segs = (Seg*)c;
  c += align256(sizeof(Seg) * (size_t)d.max_segs);
  p->seq_seg_start = (int*)c;
  c += align256(sizeof(int) * (size_t)B);
  p->seq_seg_count = (int*)c;
  c += align256(sizeof(int) * (size_t)B);
  p->wg_seg_start = (int*)c;
  c += align256(sizeof(int) * (size_t)(d.max_wg + 1));
  p->counts = (int*)c;
}

PlanJob plan_job(const PlanPtrs& p, const int32_t* kv_lens, int B, int max_kv_len, int max_pages,
                 int page, int tile, int num_splits) {
  PlanJob j;
  j.p = p;
  j.kv_lens = kv_lens;
  j.B = B;
  j.max_kv_len = max_kv_len;
  j.max_pages = max_pages;
  j.page = page;
  j.tile = tile;
  j.num_splits = num_splits;
  j.max_wg = plan_dims(B, num_splits).max_wg;
  return j;
}

hipError_t launch_plan(const PlanPtrs& p, const int32_t* kv_lens, int B, int max_kv_len,
                       int max_pages, int page, int tile, int num_splits, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s,
                     plan_job(p, kv_lens, B, max_kv_len, max_pages, page, tile, num_splits));
  return hipGetLastError();
}

hipError_t splitk_reduce_with_plan(int M, int N, int S, const float* part, long split_stride,
                                   void* out, long ldo, bool blocked, const PlanJob& job,
                                   hipStream_t s) {
  const long n = (long)M * N;
  hipLaunchKernelGGL(reduce_plan_kernel, dim3((unsigned)((n + kPlanThreads - 1) / kPlanThreads) + 1),
                     dim3(kPlanThreads), 0, s, M, N, S, part, split_stride, (__bf16*)out, ldo,
                     blocked ? 1 : 0, job);
  return hipGetLastError();
}

}  // namespace mla
