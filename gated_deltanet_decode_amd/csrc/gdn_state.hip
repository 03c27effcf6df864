// gdn_state.hip -- snapshot and restore of sequences' recurrent state.
//
// The engine must restore a recurrent state exactly from a cache, which copies
// a sequence as sections in a fixed order, and a signature over the sections'
// names, shapes and dtypes refuses a restore across models (repository
// "Architecture" page, "ModelState: sections and views").  Here a sequence
// has two sections, its fp32 state and its conv tail, and a snapshot is one
// device blob: a header, then each section for every saved sequence.
//
// Two launches per call.  A one-workgroup check validates the sequence list
// (and, for a restore, the blob's header against the expected one) and writes
// the status word; the copy launch reads that word and moves nothing unless
// it is GDN_OK.  The copy streams 16-byte units, each touched once, with
// non-temporal hints: it is bound by HBM bandwidth.
#include <cstdio>

#include "gdn.h"
#include "gdn_core.hpp"
#include "gdn_launch.hpp"

namespace gdn {

struct alignas(8) SnapHeader {
    uint32_t magic, version;
    uint64_t signature;
    uint32_t count, zero;
    uint64_t state_bytes, tail_bytes;
};

constexpr int kMaxSnapBatch = GDN_MAX_TREE_BATCH + 1;   // bitmap bits for the repeat check
static_assert(sizeof(SnapHeader) <= GDN_SNAPSHOT_HEADER_BYTES, "header fits its slot");

// restore: hdr_in is the blob's header, compared with `expect`; targets must
// be distinct.  snapshot: hdr_out receives `expect` when the list is valid.
__global__ __launch_bounds__(256) void snap_check_kernel(int B, int count, const int32_t* __restrict__ seqs,
                                                         const SnapHeader* __restrict__ hdr_in,
                                                         SnapHeader* __restrict__ hdr_out, SnapHeader expect,
                                                         int32_t* __restrict__ status) {
    __shared__ uint32_t seen[kMaxSnapBatch / 32];
    __shared__ int bad_index;
    const bool restore = hdr_in != nullptr;
    for (int i = threadIdx.x; i < (B + 31) / 32; i += blockDim.x)
        seen[i] = 0;
    if (threadIdx.x == 0)
        bad_index = 0;
    __syncthreads();
    int bad = 0;
    for (int i = threadIdx.x; i < count; i += blockDim.x) {
        const int q = seqs[i];
        if (q < 0 || q >= B) {
            bad = 1;
        } else if (restore) {
            const uint32_t bit = 1u << (q & 31);
            if (atomicOr(&seen[q >> 5], bit) & bit)
                bad = 1;   // a repeated target
        }
    }
    if (bad)
        atomicOr(&bad_index, 1);
    // The header's unused bytes are zeros.
    constexpr int kUsed = sizeof(SnapHeader) / 4;
    if (!restore && threadIdx.x >= kUsed && threadIdx.x < GDN_SNAPSHOT_HEADER_BYTES / 4)
        reinterpret_cast<uint32_t*>(hdr_out)[threadIdx.x] = 0;
    __syncthreads();
    if (threadIdx.x != 0)
        return;
    int st = bad_index ? GDN_ERR_INDEX : GDN_OK;
    if (restore && st == 0) {
        const SnapHeader h = *hdr_in;
        if (h.magic != expect.magic || h.version != expect.version || h.signature != expect.signature ||
            h.count != expect.count || h.state_bytes != expect.state_bytes || h.tail_bytes != expect.tail_bytes)
            st = GDN_ERR_SIGNATURE;
    }
    if (!restore) {
        SnapHeader h = expect;
        if (st != 0)
            h.magic = 0;   // a refused snapshot cannot be restored
        *hdr_out = h;
    }
    *status = st;
}

// One workgroup per (slot, 16 KB of the slot's sections); a thread moves four
// 16-byte units 4 KB apart.  Units [0, su) of a slot are its state, [su, su +
// tu) its tail.
template <bool RESTORE>
__global__ __launch_bounds__(256) void snap_copy_kernel(float* __restrict__ S, float* __restrict__ T,
                                                        const int32_t* __restrict__ seqs, float* __restrict__ bs,
                                                        float* __restrict__ bt, int64_t su, int64_t tu,
                                                        int wg_per_slot, const int32_t* __restrict__ status) {
    if (*status != 0)
        return;
    const int slot = blockIdx.x / wg_per_slot;
    const int64_t u0 = static_cast<int64_t>(blockIdx.x % wg_per_slot) * 1024 + threadIdx.x;
    const int64_t q = seqs[slot];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t u = u0 + 256 * k;
        if (u < su) {
            float* a = S + (q * su + u) * 4;
            float* b = bs + (slot * su + u) * 4;
            if (RESTORE)
                store_stream(a, load_stream(b));
            else
                store_stream(b, load_stream(a));
        } else if (u < su + tu) {
            float* a = T + (q * tu + (u - su)) * 4;
            float* b = bt + (slot * tu + (u - su)) * 4;
            if (RESTORE)
                store_stream(a, load_stream(b));
            else
                store_stream(b, load_stream(a));
        }
    }
}

static uint64_t fnv1a64(const char* p, size_t n) {
    uint64_t h = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < n; ++i) {
        h ^= static_cast<unsigned char>(p[i]);
        h *= 0x100000001b3ull;
    }
    return h;
}

uint64_t state_signature(const Geo& g) {
    char text[160];
    const int len = snprintf(text, sizeof text, "gdn-state-v1;state:f32[%d,%d,%d];conv_tail:%s[%d,4]", g.Hv, g.D,
                             g.D, g.bf16 ? "bf16" : "f32", g.C);
    return fnv1a64(text, static_cast<size_t>(len));
}

static int64_t state_bytes_per_seq(const Geo& g) { return static_cast<int64_t>(g.Hv) * g.D * g.D * 4; }
static int64_t tail_bytes_per_seq(const Geo& g) { return static_cast<int64_t>(g.C) * 4 * (g.bf16 ? 2 : 4); }

size_t snapshot_bytes(const Geo& g, int count) {
    return GDN_SNAPSHOT_HEADER_BYTES + static_cast<size_t>(count) * (state_bytes_per_seq(g) + tail_bytes_per_seq(g));
}

hipError_t launch_snapshot(const Geo& g, bool restore, float* S, void* tail, int count, const int32_t* seqs,
                           void* blob, int32_t* status, hipStream_t s) {
    SnapHeader expect{};
    expect.magic = GDN_SNAPSHOT_MAGIC;
    expect.version = GDN_SNAPSHOT_VERSION;
    expect.signature = state_signature(g);
    expect.count = static_cast<uint32_t>(count);
    expect.state_bytes = static_cast<uint64_t>(state_bytes_per_seq(g));
    expect.tail_bytes = static_cast<uint64_t>(tail_bytes_per_seq(g));
    SnapHeader* hdr = static_cast<SnapHeader*>(blob);
    hipLaunchKernelGGL(snap_check_kernel, dim3(1), dim3(256), 0, s, g.B, count, seqs, restore ? hdr : nullptr,
                       restore ? nullptr : hdr, expect, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t su = state_bytes_per_seq(g) / 16, tu = tail_bytes_per_seq(g) / 16;
    const int wg_per_slot = static_cast<int>((su + tu + 1023) / 1024);
    float* bs = reinterpret_cast<float*>(static_cast<char*>(blob) + GDN_SNAPSHOT_HEADER_BYTES);
    float* bt = bs + static_cast<int64_t>(count) * su * 4;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(count) * wg_per_slot)), block(256);
    if (restore)
        hipLaunchKernelGGL(snap_copy_kernel<true>, grid, block, 0, s, S, static_cast<float*>(tail), seqs, bs, bt, su,
                           tu, wg_per_slot, status);
    else
        hipLaunchKernelGGL(snap_copy_kernel<false>, grid, block, 0, s, S, static_cast<float*>(tail), seqs, bs, bt,
                           su, tu, wg_per_slot, status);
    return hipGetLastError();
}

}  // namespace gdn
