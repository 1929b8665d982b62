// w4a16_mlp.h -- gfx950 device code: a decoder layer's MLP block, gate/up +
// SwiGLU and then the down projection, in one persistent launch.
//
// The qwentin README ("How it works") lists a persistent-MLP GEMV among its
// kernels and sizes its grids to one wave of multiprocessors
// ("Performance").  Here the grid is at most one wave of workgroups, all
// resident at once.  Each workgroup runs its share of the gate/up matmul and
// writes h = bf16(silu(gate) * up) with device-scope stores; a grid barrier;
// then its share of the down projection, which stages h with device-scope
// loads.  One launch instead of two removes a launch gap per layer, and the
// down projection's weight stream starts as soon as its workgroup passes the
// barrier.
#pragma once
#include "w4a16_kernels.h"

namespace w4a16 {

struct MlpArgs {
  MatArgs up;      // phase 1: gate/up + SwiGLU, y = h
  MatArgs down;    // phase 2: down projection, x = h
  int nrb1, nwg1;  // phase 1: row blocks, workgroups (row blocks x K-slices)
  int nrb2, nwg2;  // phase 2
  int* bar;        // barrier words (see grid_barrier)
  int spin_limit;  // polls of the barrier before a workgroup gives up waiting
};

// Barrier over a grid whose workgroups are all resident, in two levels so
// that no memory word takes more than 32 atomics (same-address atomics
// serialize at the device's point of coherence): workgroup id arrives at the
// counter of its group id % 8, the last of a group at the top counter, and
// the last there advances the generation word, which the others poll.
// Words (ints, each in its own 128-byte line of the workspace):
//   bar[32 * g], g < 8   group arrival counters
//   bar[256]             top arrival counter
//   bar[288]             generation (any value; never needs initialising)
//   bar[320]             time-out flag
// Thread 0 of each workgroup, once the workgroup's stores have completed:
// reads the generation, then arrives; the last arriver of a group resets the
// group's counter (all its members have arrived), the last arriver at the top
// resets the top counter and advances the generation; every other workgroup
// polls the generation (sleeping between polls), at most spin_limit polls --
// after that it sets the time-out flag and goes on, so every workgroup still
// runs to its end and the counters are still reset (the call's result is then
// undefined and the flag says so).  The generation cannot advance before the
// reader arrives, so reading it first is safe.
constexpr int kBarGroupStride = 32, kBarTop = 256, kBarGen = 288, kBarFlag = 320;

W4A16_DEV int atomic_add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
W4A16_DEV int load_agent(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
W4A16_DEV void store_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

W4A16_DEV void grid_barrier(int* bar, int id, int nwg, int spin_limit) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __syncthreads();                // ... and so have every other wave's
  if (threadIdx.x == 0) {
    const int g = id & 7;
    const int in_group = (nwg - g + 7) >> 3;  // workgroups with this id % 8
    const int groups = nwg < 8 ? nwg : 8;
    const int gen = load_agent(bar + kBarGen);
    bool released = false;
    if (atomic_add_agent(bar + kBarGroupStride * g, 1) == in_group - 1) {
      store_agent(bar + kBarGroupStride * g, 0);
      if (atomic_add_agent(bar + kBarTop, 1) == groups - 1) {
        store_agent(bar + kBarTop, 0);
        store_agent(bar + kBarGen, gen + 1);
        released = true;
      }
    }
    int polls = 0;
    while (!released && load_agent(bar + kBarGen) == gen) {
      if (++polls > spin_limit) {
        store_agent(bar + kBarFlag, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Workgroup id -> (row block, K-slice) of a phase: id = ks * nrb + rb.
W4A16_DEV void phase_coords(int id, int nrb, int& rb, int& ks) {
  ks = id / nrb;
  rb = id - ks * nrb;
}

// M <= 2: both phases on the VALU kernel body (L1, L2 lanes per weight row).
template <int MT, int L1, int L2, int D, int LB>
__global__ void __launch_bounds__(LB) k_mlp_valu(MlpArgs m) {
  const int id = blockIdx.x;
  int rb, ks;
  if (id < m.nwg1) {
    phase_coords(id, m.nrb1, rb, ks);
    gemm_valu<MT, L1, D, kEpiSwiglu, LB, kCoStoreY>(m.up, rb, ks, m.nrb1);
  }
  grid_barrier(m.bar, id, gridDim.x, m.spin_limit);
  if (id < m.nwg2) {
    phase_coords(id, m.nrb2, rb, ks);
    gemm_valu<MT, L2, D, kEpiPlain, LB, kCoLoadX>(m.down, rb, ks, m.nrb2);
  }
}

// 3 <= M <= 32: both phases on the MFMA kernel body (P passes of 4 rows).
template <int P, int D, int LB>
__global__ void __launch_bounds__(LB) k_mlp_mfma(MlpArgs m) {
  const int id = blockIdx.x;
  int rb, ks;
  if (id < m.nwg1) {
    phase_coords(id, m.nrb1, rb, ks);
    gemm_mfma<P, 1, D, kEpiSwiglu, LB, kCoStoreY>(m.up, rb, ks, m.nrb1);
  }
  grid_barrier(m.bar, id, gridDim.x, m.spin_limit);
  if (id < m.nwg2) {
    phase_coords(id, m.nrb2, rb, ks);
    gemm_mfma<P, 1, D, kEpiPlain, LB, kCoLoadX>(m.down, rb, ks, m.nrb2);
  }
}

}  // namespace w4a16
