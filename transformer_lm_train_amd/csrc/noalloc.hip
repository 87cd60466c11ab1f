// Entry points that allocate nothing, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid it).  Their kernels' scratch lives in a file-scope device array
// that every GPU the library runs on holds until the process ends; its
// address on each device is looked up once, with that device current, and
// only that address is ever handed to a kernel.
#include <mutex>

#include "../../include/gpt2.h"
#include "kernels.h"

namespace {

// The attention backward's per-row statistics (D = rowsum(dO o O), then the
// base-2 log-sum-exp of every query row) for up to 2^20 rows of B*NH*T:
// 8 MiB per device.
constexpr size_t SCRATCH_FLOATS = (size_t)2 << 20;
__device__ __align__(256) float scratch[SCRATCH_FLOATS];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
float* g_scratch[MAX_DEVICES];  // device address of `scratch` on each device, once looked up

// The address of `scratch` on the current device (looked up on the first call there).
int scratch_on_current_device(float** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return gpt2_report_error(GPT2_EIO, "no usable current HIP device");
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return gpt2_report_error(GPT2_EIO, "hipGetSymbolAddress of the static scratch buffer failed");
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return GPT2_OK;
}

}  // namespace

extern "C" int gpt2_attention_bwd_noalloc(void* hip_stream, void* dqkv, const void* dout, const void* qkv,
                                          const void* out, const float* lse, int B, int T, int C, int NH) {
    if (!dqkv || !dout || !qkv || !out || !lse) return gpt2_report_error(GPT2_EINVAL, "NULL array argument");
    if (B <= 0 || T <= 0 || NH <= 0 || C <= 0 || C % NH || C / NH != 64 || T % 64)
        return gpt2_report_error(GPT2_EINVAL, "need B, T, NH > 0, head size C/NH = 64 and T a multiple of 64");
    const size_t need = flash_attention_bwd_ws_floats(B, T, NH);
    if (need > SCRATCH_FLOATS)
        return gpt2_report_error(GPT2_EINVAL, "B*NH*T exceeds the 1048576 attention rows the static scratch holds");
    float* ws = nullptr;
    if (int rc = scratch_on_current_device(&ws)) return rc;
    const hipError_t e = flash_attention_bwd(static_cast<bf16*>(dqkv), static_cast<const bf16*>(dout),
                                             static_cast<const bf16*>(qkv), static_cast<const bf16*>(out), lse, ws, B,
                                             T, C, NH, nullptr, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return gpt2_report_error(GPT2_EIO, hipGetErrorString(e));
    return GPT2_OK;
}
