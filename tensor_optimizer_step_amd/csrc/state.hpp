// Device-resident optimizer state shared by the host code and the kernels.
#pragma once

#include <cstdint>

#include "somaopt.h"

namespace somaopt {

// Per-group constants of the pending update, produced in fp64 by the norm
// pass's last workgroup and rounded once to fp32 for the elementwise update.
struct GroupConst {
    float step_size;        // lr / (1 - beta1^t)
    float inv_sqrt_bc2;     // 1 / sqrt(1 - beta2^t)
    float lr_wd;            // lr * weight_decay (decoupled decay)
    float beta1;
    float one_minus_beta1;
    float beta2;
    float one_minus_beta2;
    float eps;
};
static_assert(sizeof(GroupConst) == 32, "GroupConst layout");

struct DevState {
    somaopt_stats stats;           // public statistics block (first member)
    float grad_scale_f32;          // clip_coef / grad_divisor, rounded to fp32
    int32_t n_groups;
    double max_norm;
    double grad_divisor;
    int64_t step[SOMAOPT_MAX_GROUPS];         // completed (or pending) updates per group
    somaopt_group hyper[SOMAOPT_MAX_GROUPS];  // current hyperparameters
    GroupConst gconst[SOMAOPT_MAX_GROUPS];    // constants of the pending update
    somaopt_schedule sched[SOMAOPT_MAX_GROUPS];   // on-device lr schedules (kind 0: none)
};

// Kernel-argument carrier for somaopt_set_groups (passed by value).
struct GroupArgs {
    int32_t n;
    int32_t pad;
    somaopt_group g[SOMAOPT_MAX_GROUPS];
};

// Kernel-argument carrier for somaopt_set_schedules (passed by value).
struct ScheduleArgs {
    int32_t n;
    int32_t pad;
    somaopt_schedule s[SOMAOPT_MAX_GROUPS];
};

}  // namespace somaopt
