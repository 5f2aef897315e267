// Test helper (not part of the library): a kernel that holds CUs for a
// bounded time, so a test can run a verify call while only part of the GPU
// is free. Each workgroup takes a CU's whole LDS and 1024 threads, sleeps a
// fixed number of rounds and exits.
#include <hip/hip_runtime.h>

__global__ __launch_bounds__(1024) void occupy_kernel(unsigned rounds, unsigned* out) {
    extern __shared__ unsigned char lds[];
    for (unsigned i = 0; i < rounds; ++i) __builtin_amdgcn_s_sleep(127);
    if (threadIdx.x == 0) {
        lds[0] = 1;
        out[blockIdx.x] = lds[0];
    }
}

// blocks workgroups, each holding one CU's LDS; rounds of s_sleep(127) each
// (about 3 us per round). out: int32 [blocks] device buffer. Returns 0 or -1.
extern "C" int sv_test_occupy(int blocks, unsigned rounds, unsigned* out, void* stream) {
    int dev = 0, lds = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipFuncSetAttribute((const void*)occupy_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            lds) != hipSuccess) {
        return -1;
    }
    hipLaunchKernelGGL(occupy_kernel, dim3(blocks), dim3(1024), (size_t)lds,
                       static_cast<hipStream_t>(stream), rounds, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
