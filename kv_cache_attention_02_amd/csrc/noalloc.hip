// Library-held scratch for wmk_chunk_attention_noalloc: the split tail's fp32
// partial results live in one file-scope device array instead of caller
// memory, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  The host-side name `scratch` is only a
// stand-in for that address: the device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and kept in a fixed
// per-device table; every kernel argument uses the looked-up address.
//
// Every call on one GPU shares that GPU's array, and the array keeps the last
// call's contents.  Nothing in it needs to start at zero: each split piece
// writes all of its partial rows before the merge kernel, later on the same
// stream, reads them.  Calls that overlap on one GPU (different streams, or
// different host threads without ordering) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wmk_internal.h"

namespace wmk {
namespace {

// 256 split pieces -- one per resident workgroup of the 8-wave attention kernel
// on a 256-CU MI355X -- of 256 query rows x 128 dims in fp32, plus (max, sum)
// per row; the same bytes hold the 512 pieces of 128 rows of the 4-wave kernel
// (two workgroups per CU).
constexpr size_t kScratchBytes = (size_t)256 * (256 * 128 + 2 * 256) * sizeof(float);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace wmk
