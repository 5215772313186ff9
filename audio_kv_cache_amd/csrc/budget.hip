// budget.hip -- the budget kernel: one 1024-thread workgroup per budget
// pool, the pool's arithmetic in budget.h.
#include "budget.h"

__global__ __launch_bounds__(1024) void kvc_budget_kernel(KvcDesc D, const float* S,
                                                          int32_t* budgets, int64_t* offsets) {
  __shared__ __attribute__((aligned(16))) KvcBudgetSmem sm;
  kvc_budget_pool<1024>(D, S, budgets, offsets, (int)blockIdx.x, sm);
}

hipError_t kvc_launch_budget(const KvcDesc& D, const float* S, int32_t* budgets,
                             int64_t* offsets, hipStream_t st) {
  hipLaunchKernelGGL(kvc_budget_kernel, dim3(D.n_seq * (D.upseq / D.pool_size)),
                     dim3(1024), 0, st, D, S, budgets, offsets);
  return hipGetLastError();
}
