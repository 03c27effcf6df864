// gdn_launch.hpp -- host-side launchers of the kernels, called by the C ABI
// after it has validated every argument.  Each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct Geo {
    int B, Hk, Hv, D, C;
    bool bf16;
};

hipError_t launch_conv_update(const Geo& g, const void* x, void* tail, const void* w, float* y, hipStream_t s);
hipError_t launch_decode(const Geo& g, float* S, const float* y, const float* a, const float* b, float* o,
                         hipStream_t s);
hipError_t launch_token(const Geo& g, float* S, const void* tail_in, void* tail_out, const void* w, const void* x,
                        const float* a, const float* b, float* o, hipStream_t s);
// The per-channel-decay step: a is [B][Hv][D] (one forget-gate input per key channel).
hipError_t launch_kda_decode(const Geo& g, float* S, const float* y, const float* a, const float* b, float* o,
                             hipStream_t s);
hipError_t launch_kda_token(const Geo& g, float* S, const void* tail_in, void* tail_out, const void* w,
                            const void* x, const float* a, const float* b, float* o, hipStream_t s);
hipError_t launch_tree_tables(int n, const int32_t* parent, int32_t* depth, int32_t* order, int32_t* status,
                              hipStream_t s);
size_t tree_ws_bytes(int B, int n, int Hk, int Hv, int D);
hipError_t launch_tree_verify(const Geo& g, const float* S, const void* tail, const void* w, int n,
                              const int32_t* parent, const void* x, const float* a, const float* b, float* o,
                              int32_t* status, void* ws, hipStream_t s);
hipError_t launch_tree_verify_ut(const Geo& g, const float* S, const void* tail, const void* w, int n,
                                 const int32_t* parent, const void* x, const float* a, const float* b, float* o,
                                 int32_t* status, void* ws, hipStream_t s);
hipError_t launch_block(const Geo& g, bool commit, float* S, void* tail, const void* w, int k, const void* x,
                        const float* a, const float* b, const int32_t* accepted, float* o, int32_t* status, void* ws,
                        bool prepared, hipStream_t s);
hipError_t launch_commit(const Geo& g, float* S, void* tail, const void* w, int n, const int32_t* parent,
                         const void* x, const float* a, const float* b, int L, const int32_t* path, float* o,
                         int32_t* status, void* ws, hipStream_t s);
uint64_t state_signature(const Geo& g);
size_t snapshot_bytes(const Geo& g, int count);
hipError_t launch_snapshot(const Geo& g, bool restore, float* S, void* tail, int count, const int32_t* seqs,
                           void* blob, int32_t* status, hipStream_t s);
size_t prefill_workspace_bytes(const Geo& g, int T);
hipError_t launch_prefill(const Geo& g, float* S, void* tail, const void* w, int T, const void* x, const float* a,
                          const float* b, float* o, void* ws, hipStream_t s);

size_t self_check_ws_bytes(const Geo& g);
hipError_t launch_self_check(const Geo& g, void* ws, uint32_t seed, int perturb, int32_t* result, hipStream_t s);
// Device address of the library-held scratch array on the current device.
hipError_t noalloc_scratch(void** out);

}  // namespace gdn
