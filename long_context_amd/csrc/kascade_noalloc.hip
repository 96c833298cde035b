// kascade_reuse_decode_noalloc: kascade_reuse_decode without a caller
// workspace, for callers that cannot allocate device memory (code under graph
// capture, tight serving loops, harnesses that forbid allocation). Its
// scratch -- the gather's arrival counters and partials -- is a file-scope
// device array, one copy per GPU, held until the process ends.
#include <mutex>
#include <vector>

#include "api_internal.hpp"

namespace {

// The array's size, the largest workspace this entry point serves.
constexpr size_t kScratchBytes = KASCADE_NOALLOC_SCRATCH_BYTES;

// Zero at load. Host code never passes this name to a kernel or a copy: on
// the host it is a stand-in, not a device address. Its device address on the
// current GPU comes from hipGetSymbolAddress (scratch_on_device below).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void clear_scratch(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchTable {
  std::mutex mu;
  std::vector<char*> address;  // per device; null until set up
};

ScratchTable& scratch_table() {
  static ScratchTable t;
  return t;
}

// Device address of `scratch` on the current GPU. Set-up, once per GPU at its
// first call: look the address up and clear the array with a kernel on `s`
// (arrival counters must start at zero; every call leaves them zero after).
hipError_t scratch_on_device(hipStream_t s, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  ScratchTable& t = scratch_table();
  std::lock_guard<std::mutex> lock(t.mu);
  if ((int)t.address.size() <= dev) t.address.resize(dev + 1, nullptr);
  if (!t.address[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(clear_scratch, dim3(256), dim3(256), 0, s, static_cast<uint4*>(ptr),
                       kScratchBytes / sizeof(uint4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    t.address[dev] = static_cast<char*>(ptr);
  }
  *out = t.address[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int kascade_reuse_decode_noalloc(const kascade_problem* p, const void* q, const void* k,
                                            const void* v, const int32_t* idx, void* out, void* stream) {
  int rc = kascade::reuse_decode_check(p, q, k, v, idx, out);
  if (rc) return rc;
  if (kascade_workspace_bytes(p, KASCADE_OP_REUSE_DECODE) > kScratchBytes) return KASCADE_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  if (scratch_on_device(s, &ws) != hipSuccess) return KASCADE_ERR_HIP;
  return kascade::reuse_decode_enqueue(p, q, k, v, idx, out, ws, s);
}
