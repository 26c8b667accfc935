// Host launchers of the In-Place ABN kernels.  They enqueue on `s` and return;
// arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>

#include "plan.hpp"

namespace iabn {

void launch_forward_stats(const Plan& pl, const void* x, const float* gamma, const float* beta,
                          float* running_mean, float* running_var, float* save_mean,
                          float* save_invstd, float eps, float momentum, void* ws, hipStream_t s);

void launch_forward_apply(const Plan& pl, void* x, int act, float a, void* ws, hipStream_t s);

void launch_forward_eval(const Plan& pl, void* x, const float* gamma, const float* beta,
                         const float* rm, const float* rv, float eps, int act, float a,
                         hipStream_t s);

void launch_backward_reduce(const Plan& pl, const void* y, const void* dy, const float* gamma,
                            const float* beta, const float* invstd, float* dgamma, float* dbeta,
                            int act, float a, void* ws, hipStream_t s);

// Backward through the inference forward with dgamma/dbeta: one pass over y and dy
// writes dx (it needs no reduction) and the partial sums, then the sums are
// finished.
void launch_backward_eval_grads(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* running_var,
                                float eps, float* dgamma, float* dbeta, int act, float a,
                                void* ws, hipStream_t s);

// dx constants of the backward through the inference forward, without the sums.
void launch_eval_consts(const Plan& pl, const float* gamma, const float* beta,
                        const float* running_var, float eps, void* ws, hipStream_t s);

void launch_backward_apply(const Plan& pl, const void* y, const void* dy, void* dx, int act,
                           float a, void* ws, hipStream_t s);

// Optimized checkpointing (the block keeps xhat): the backward sums read from
// xhat, leaving dgamma, dbeta and the dx constants {A, B, Cc, beta} with
// dx = A*dz + B*xhat + Cc.
void launch_backward_reduce_xhat(const Plan& pl, const void* xhat, const void* dy,
                                 const float* gamma, const float* beta, const float* invstd,
                                 float* dgamma, float* dbeta, int act, float a, void* ws,
                                 hipStream_t s);

// xhat written over x and y = act(gamma*xhat + beta) into y, from the constants
// launch_forward_stats left in the workspace and its save_invstd.
void launch_ckpt_forward_apply(const Plan& pl, void* x, void* y, const float* gamma,
                               const float* beta, const float* invstd, int act, float a, void* ws,
                               hipStream_t s);

// y = act(gamma*xhat + beta).
void launch_ckpt_recompute(const Plan& pl, const void* xhat, void* y, const float* gamma,
                           const float* beta, int act, float a, hipStream_t s);

// dx from xhat and dy, with the constants launch_backward_reduce_xhat left.
void launch_ckpt_dx(const Plan& pl, const void* xhat, const void* dy, void* dx,
                    const float* gamma, const float* beta, int act, float a, void* ws,
                    hipStream_t s);

}  // namespace iabn
