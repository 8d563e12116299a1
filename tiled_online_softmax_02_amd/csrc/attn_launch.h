// attn_launch.h -- internal interface between the C ABI (attn_api.hip) and the
// kernel files.  Arguments have already been validated when these are called.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// Shape of the device the launch goes to: compute units and XCDs (each XCD has its own L2; consecutive
// workgroups are dispatched to the XCDs in turn).
struct DeviceShape {
    int cus, nx;
};

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, H, Hk, Nq, Nk, d, causal;  // H query heads, Hk K/V heads; Nq query rows, Nk key rows per head
    float scale;
    void *stream;
    DeviceShape dev;
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *delta;
    int B, H, Hk, Nq, Nk, d, causal;  // H query heads, Hk K/V heads; Nq query rows, Nk key rows per head
    float scale;
    void *stream;
    DeviceShape dev;
};

// Forward pass on e4m3 inputs with per-head scales (d = 64 or 128).
struct Fp8FwdArgs {
    const void *q, *k, *v;                                 // e4m3 codes
    const float *descale_q, *descale_k, *descale_v;        // [B*H], [B*Hk], [B*Hk]
    void *o;                                               // bf16
    float *lse;
    int B, H, Hk, Nq, Nk, d, causal;
    float scale;
    void *stream;
    DeviceShape dev;
};

hipError_t launch_fwd(const FwdArgs &a);
hipError_t launch_fwd_fp8(const Fp8FwdArgs &a);
// Split-key forward: partial pieces into `workspace` (fwd_split_workspace_bytes), then the merge.
hipError_t launch_fwd_split(const FwdArgs &a, int n_splits, void *workspace);
hipError_t launch_bwd_preprocess(const BwdArgs &a);
hipError_t launch_bwd_dkdv(const BwdArgs &a);
hipError_t launch_bwd_dq(const BwdArgs &a);
// The dQ kernel that also forms D of its rows from O and dO and writes it to a.delta (bitwise
// what the preprocess kernel writes); launched before the dK/dV kernel, which reads D.
bool bwd_dq_fuses_delta(int d);
hipError_t launch_bwd_dq_delta(const BwdArgs &a);

long long fwd_grid_size(int B, int H, int Nq);
long long fwd_split_grid_size(int B, int H, int Nq, int n_splits);
long long fwd_split_workspace_bytes(int B, int H, int Nq, int d, int n_splits);
int fwd_split_default(int B, int H, int Hk, int Nq, int Nk, int d);
long long bwd_dkdv_grid_size(int B, int Hk, int Nk);
long long bwd_dq_grid_size(int B, int H, int Nq);

}  // namespace attn
