// Measurement program (not part of libtclora): what a grid-wide wait costs
// inside one launch on this GPU, against an empty launch of the same grid.
// It backs the choice of two launches (shrink, then expand) for the decode
// step over one launch whose workgroups wait for every shrink result.
//
// Each workgroup of 512 threads writes `dirty` floats (like the shrink's z
// rows), then thread 0 arrives and waits; the wait polls at most spin_limit
// times, so every wave exits whatever happens.  Forms:
//   0  no wait (the empty launch)
//   1  one device-wide counter; release add, acquire polls
//   2  per-XCD counters (workgroup b runs on XCD b % 8), the last arrival of
//      an XCD adds to the device-wide counter; release adds, acquire polls
//   3  as 2, with relaxed polls and one acquire fence after the loop (the
//      cheapest form that still publishes the written data)
//   4  as 2 with relaxed adds and polls (publishes nothing: a lower bound)
//   5  as 4 over a three-level tree (8 workgroups a leaf counter)
//
// Build and run (one GPU):
//   hipcc -O3 --offload-arch=gfx950 probe_grid_wait.hip -o probe_grid_wait
//   ./probe_grid_wait <workgroups> <floats written per workgroup>
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CK(x)                                                                           \
  do {                                                                                  \
    hipError_t e = (x);                                                                 \
    if (e != hipSuccess) {                                                              \
      printf("HIP error %s at line %d\n", hipGetErrorString(e), __LINE__);              \
      exit(1);                                                                          \
    }                                                                                   \
  } while (0)

// ctr words: [16 x] per-XCD counters, [128] device-wide, [160] timeout flag,
// [1024 + 16 l] leaf counters
template <int FORM>
__global__ __launch_bounds__(512) void grid_wait(unsigned *ctr, float *data, int G,
                                                 int spin_limit, int dirty) {
  __shared__ int ok;
  const int b = blockIdx.x, xcd = b & 7;
  for (int i = threadIdx.x; i < dirty; i += 512) data[int64_t(b) * dirty + i] = float(i);
  __syncthreads();
  if (FORM == 0) return;
  if (threadIdx.x == 0) {
    unsigned target = 8;
    const unsigned nx = (G - xcd + 7) / 8;
    if (FORM == 1) {
      __hip_atomic_fetch_add(&ctr[128], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      target = G;
    } else if (FORM == 2 || FORM == 3) {
      const unsigned v =
          __hip_atomic_fetch_add(&ctr[xcd * 16], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      if (v == nx - 1)
        __hip_atomic_fetch_add(&ctr[128], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else if (FORM == 4) {
      const unsigned v =
          __hip_atomic_fetch_add(&ctr[xcd * 16], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v == nx - 1)
        __hip_atomic_fetch_add(&ctr[128], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const int k = b >> 3;
      const unsigned nleaf = (nx + 7) / 8, in_leaf = min(8u, nx - unsigned(k & ~7));
      unsigned *lc = &ctr[1024 + (xcd * 64 + (k >> 3)) * 16];
      if (__hip_atomic_fetch_add(lc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          in_leaf - 1) {
        if (__hip_atomic_fetch_add(&ctr[xcd * 16], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) == nleaf - 1)
          __hip_atomic_fetch_add(&ctr[128], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    int it = 0;
    if (FORM <= 2) {
      while (__hip_atomic_load(&ctr[128], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (++it > spin_limit) break;
        __builtin_amdgcn_s_sleep(1);
      }
    } else {
      while (__hip_atomic_load(&ctr[128], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (++it > spin_limit) break;
        __builtin_amdgcn_s_sleep(1);
      }
      __atomic_thread_fence(__ATOMIC_ACQUIRE);
    }
    ok = it <= spin_limit;
    if (!ok) atomicOr(&ctr[160], 1u);
  }
  __syncthreads();
  if (ok) data[int64_t(b) * dirty] += 1.f;
}

template <int FORM>
static void launch(unsigned *ctr, float *data, int G, int dirty) {
  hipLaunchKernelGGL(grid_wait<FORM>, dim3(G), dim3(512), 0, 0, ctr, data, G, 100000, dirty);
}

int main(int argc, char **argv) {
  const int G = argc > 1 ? atoi(argv[1]) : 512;
  const int dirty = argc > 2 ? atoi(argv[2]) : 1024;
  if (G < 8 || G > 1024 || dirty < 1 || dirty > (1 << 20)) {
    printf("workgroups in [8, 1024], floats in [1, 2^20]\n");
    return 2;
  }
  const size_t ctr_words = 65536;
  unsigned *ctr;
  float *data;
  CK(hipMalloc(&ctr, ctr_words * 4));
  CK(hipMalloc(&data, size_t(G) * dirty * 4));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  for (int form = 0; form < 6; ++form) {
    const int reps = 50;
    float best = 1e9f, sum = 0.f;
    unsigned timeouts = 0;
    for (int r = 0; r < reps + 5; ++r) {
      CK(hipMemset(ctr, 0, ctr_words * 4));
      CK(hipDeviceSynchronize());
      CK(hipEventRecord(e0, 0));
      switch (form) {
        case 0: launch<0>(ctr, data, G, dirty); break;
        case 1: launch<1>(ctr, data, G, dirty); break;
        case 2: launch<2>(ctr, data, G, dirty); break;
        case 3: launch<3>(ctr, data, G, dirty); break;
        case 4: launch<4>(ctr, data, G, dirty); break;
        default: launch<5>(ctr, data, G, dirty); break;
      }
      CK(hipGetLastError());
      CK(hipEventRecord(e1, 0));
      CK(hipEventSynchronize(e1));
      float ms;
      CK(hipEventElapsedTime(&ms, e0, e1));
      unsigned flag;
      CK(hipMemcpy(&flag, ctr + 160, 4, hipMemcpyDeviceToHost));
      timeouts |= flag;
      if (r >= 5) {
        best = ms < best ? ms : best;
        sum += ms;
      }
    }
    printf("workgroups=%d floats=%d form=%d best %.2f us mean %.2f us timeouts=%u\n", G, dirty,
           form, best * 1e3, sum / reps * 1e3, timeouts);
  }
  CK(hipFree(ctr));
  CK(hipFree(data));
  return 0;
}
