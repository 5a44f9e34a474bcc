// Persistent small-batch decode: every layer's five fused ops in one kernel.
//
// At batch 1 a decode step is a chain of 140 small dependent kernels (five
// per layer; rvLLM post on discuss.pytorch.kr, section "CUDA 그래프
// 리플레이", and its optimisation history: fewer launches and cross-layer
// fusion).  Here one kernel runs the layer loop itself: a grid of resident
// workgroups (one or two per CU) walks the phases QKV + RoPE + append,
// attention, O + residual, RMSNorm + gate/up + SiLU*mul, down + residual of
// every layer, with a grid-wide barrier between phases.  Each phase runs the
// same device bodies as the per-op kernels (gemv_body, attn_body) over the
// same virtual blocks, so the result equals the per-op path bit for bit.
//
// Memory between phases: the XCDs' L2 caches are not coherent with each
// other, so every activation a phase hands to the next (q, the attention
// output, the hidden state, the SiLU*mul activation) is written and read with
// agent-scope accesses (the bodies' COH mode); the new token's k and v are
// already stored write-through; weights are read-only.  The barrier: each
// workgroup waits for its own stores, then arrives in two levels with
// agent-scope atomics (its group of workgroups, then, for the last of a group,
// the root), and the last to reach the root publishes the barrier's number in
// a release word that every workgroup polls.  32 groups keep any one counter
// to a few dozen serialised atomics: one counter for the whole grid cost
// about 8 us per barrier at 512 workgroups, the two levels about 2 us.  A
// barrier that does not complete within 250 ms (a grid that could not be
// resident at once) sets an error flag and lets the kernel finish, so no wait
// can hang; the flag makes the following barriers return at once.
#include "attn_body.h"
#include "gemv_body.h"

namespace pkv {
namespace {

constexpr int kMaxPersistLayers = 64;

struct PParams {
  LinArgs qkv, o, gu, down;  // arguments of layer 0; per-layer weights from `layers`
  SplitParams sp;            // attention of layer 0
  const PersistLayer* layers;
  const unsigned char* k_pool0;
  size_t pool_stride;  // bytes from one layer's K pool to the next layer's
  size_t v_off;        // bytes from a layer's K pool to its V pool
  float rope_ks[kMaxPersistLayers], rope_vs[kMaxPersistLayers];  // append scales (1 for f16)
  float attn_sl2[kMaxPersistLayers], attn_vs[kMaxPersistLayers];   // attention score / V scales
  int n_layers;
  int nb_qkv, nb_attn, nb_o, nb_gu, nb_down;  // virtual blocks of each phase
  int cfg_hidden, cfg_gu, attn_nt;            // body variants (see persistent_config)
  unsigned* barrier;  // kBarrierWords words, zero at launch; word 0 is the error flag
  unsigned long long timeout_ticks;  // wall-clock ticks a barrier may wait
};

// Barrier words (unsigned, each in a 256-byte line of its own, zero at launch):
// [0] error flag, [64] release (number of the last completed barrier),
// [128] root count, [192 + 64 g] count of group g.
constexpr int kBarrierGroups = 32;
constexpr int kBarrierWords = 192 + 64 * kBarrierGroups;
static_assert(kGemmMaxCounters >= kBarrierWords, "barrier words live in the split-K counter area");

__device__ __forceinline__ unsigned ld_word(unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned arrive(unsigned* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier number n (1, 2, ... within one launch).
__device__ __forceinline__ void grid_sync(const PParams& pp, unsigned n) {
  wait_vmcnt<0>();  // this wave's stores (and loads) have completed
  __syncthreads();
  unsigned* w = pp.barrier;
  if (threadIdx.x == 0 && !ld_word(w)) {
    const unsigned G = gridDim.x, g = blockIdx.x % kBarrierGroups;
    const unsigned members = (G - g + kBarrierGroups - 1) / kBarrierGroups;
    const unsigned groups = G < (unsigned)kBarrierGroups ? G : (unsigned)kBarrierGroups;
    if (arrive(w + 192 + 64 * g) + 1 == n * members && arrive(w + 128) + 1 == n * groups)
      __hip_atomic_store(w + 64, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long t0 = wall_clock64();
    while (ld_word(w + 64) < n) {
      __builtin_amdgcn_s_sleep(1);
      if (ld_word(w)) break;  // another workgroup timed out
      if (wall_clock64() - t0 > pp.timeout_ticks) {
        __hip_atomic_store(w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// The batch-1 GEMV variants the kernel carries: projections over the hidden
// size (QKV, O) take 128 lanes per row with 2 or 4 chunk steps (cfg_hidden
// 0 / 1); gate/up takes 32 or 64 lanes with 8 steps (cfg_gu 0 / 1); the down
// projection 256 lanes with 8 steps.
template <int EPI, bool NORM>
__device__ __forceinline__ void gemv_hidden(int cfg, const LinArgs& a, int vb) {
  if (cfg == 0)
    gemv_body<128, 1, 2, EPI, NORM, true>(a, vb);
  else
    gemv_body<128, 1, 4, EPI, NORM, true>(a, vb);
}

template <bool FP8>
__global__ void __launch_bounds__(256, 2) persist_kernel(PParams pp) {
  const int G = gridDim.x, wg = blockIdx.x;
  unsigned phase = 0;  // barriers passed
  for (int l = 0; l < pp.n_layers; ++l) {
    const PersistLayer L = pp.layers[l];
    unsigned char* kp = const_cast<unsigned char*>(pp.k_pool0) + (size_t)l * pp.pool_stride;
    unsigned char* vp = kp + pp.v_off;
    {  // 1. RMSNorm + QKV + bias, RoPE, q out, new k and v into the cache
      LinArgs a = pp.qkv;
      a.W = L.w_qkv;
      a.gain = L.w_in;
      a.bias = L.b_qkv;
      a.rope.k_pool = kp;
      a.rope.v_pool = vp;
      a.rope.k_scale = pp.rope_ks[l];
      a.rope.v_scale = pp.rope_vs[l];
      for (int vb = wg; vb < pp.nb_qkv; vb += G) {
        gemv_hidden<EPI_ROPE, true>(pp.cfg_hidden, a, vb);
        __syncthreads();
      }
    }
    grid_sync(pp, ++phase);
    {  // 2. paged GQA attention (split partitions merged by the last to finish)
      SplitParams sp = pp.sp;
      sp.k_pool = kp;
      sp.v_pool = vp;
      sp.scale_log2 = pp.attn_sl2[l];
      sp.v_scale = pp.attn_vs[l];
      for (int vb = wg; vb < pp.nb_attn; vb += G) {
        if (pp.attn_nt == 2)
          attn_body<128, FP8, 2, 4, true>(sp, vb);
        else
          attn_body<128, FP8, 4, 4, true>(sp, vb);
        __syncthreads();
      }
    }
    grid_sync(pp, ++phase);
    {  // 3. O projection + residual add
      LinArgs a = pp.o;
      a.W = L.w_o;
      for (int vb = wg; vb < pp.nb_o; vb += G) {
        gemv_hidden<EPI_RESID, false>(pp.cfg_hidden, a, vb);
        __syncthreads();
      }
    }
    grid_sync(pp, ++phase);
    {  // 4. RMSNorm + gate/up + SiLU*mul
      LinArgs a = pp.gu;
      a.W = L.w_gu;
      a.gain = L.w_post;
      for (int vb = wg; vb < pp.nb_gu; vb += G) {
        if (pp.cfg_gu == 0)
          gemv_body<32, 1, 8, EPI_SILU, true, true>(a, vb);
        else
          gemv_body<64, 1, 8, EPI_SILU, true, true>(a, vb);
        __syncthreads();
      }
    }
    grid_sync(pp, ++phase);
    {  // 5. down projection + residual add
      LinArgs a = pp.down;
      a.W = L.w_down;
      for (int vb = wg; vb < pp.nb_down; vb += G) {
        gemv_body<256, 1, 8, EPI_RESID, false, true>(a, vb);
        __syncthreads();
      }
    }
    if (l + 1 < pp.n_layers) grid_sync(pp, ++phase);
  }
}

// Workgroups of the grid: the CUs times the workgroups of the kernel one CU
// holds at once (at most 2), per device, queried once.
int persistent_grid(bool fp8) {
  static int cached[2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int& g = cached[fp8][dev];
  if (g == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const hipError_t e = fp8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, persist_kernel<true>, 256, 0)
                             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, persist_kernel<false>, 256, 0);
    if (e != hipSuccess) return 0;
    g = cus * std::min(per_cu, 2);
    if (g <= 0) g = -1;
  }
  return g > 0 ? g : 0;
}

}  // namespace

bool persistent_config(const PersistArgs& a, int* cfg_hidden, int* cfg_gu) {
  if (a.n_layers < 1 || a.n_layers > kMaxPersistLayers) return false;
  if (a.qkv.M != 1 || a.attn.head_dim != 128) return false;
  if (a.plan.waves != 4 || (a.plan.nt != 2 && a.plan.nt != 4)) return false;
  int l_qkv, u_qkv, l_o, u_o, l_gu, u_gu, l_dn, u_dn;
  gemv_config(a.qkv.n_out, a.qkv.K, &l_qkv, &u_qkv);
  gemv_config(a.o.n_out, a.o.K, &l_o, &u_o);
  gemv_config(a.gu.n_out, a.gu.K, &l_gu, &u_gu);
  gemv_config(a.down.n_out, a.down.K, &l_dn, &u_dn);
  if (l_qkv != 128 || l_o != 128 || u_qkv != u_o || (u_qkv != 2 && u_qkv != 4)) return false;
  if ((l_gu != 32 && l_gu != 64) || u_gu != 8 || l_dn != 256 || u_dn != 8) return false;
  *cfg_hidden = u_qkv == 2 ? 0 : 1;
  *cfg_gu = l_gu == 32 ? 0 : 1;
  return persistent_grid(a.attn.fp8) > 0;
}

hipError_t launch_persistent_layers(const PersistArgs& a, hipStream_t s) {
  PParams pp{};
  int cfg_hidden = 0, cfg_gu = 0;
  if (!persistent_config(a, &cfg_hidden, &cfg_gu)) return hipErrorInvalidValue;
  pp.qkv = a.qkv;
  pp.o = a.o;
  pp.gu = a.gu;
  pp.down = a.down;
  pp.sp = make_split_params(a.attn, a.plan);
  pp.layers = a.layers;
  pp.k_pool0 = static_cast<const unsigned char*>(a.attn.k_pool);
  pp.pool_stride = a.pool_stride;
  pp.v_off = a.v_off;
  for (int l = 0; l < a.n_layers; ++l) {
    const bool fp8 = a.attn.fp8;
    pp.rope_ks[l] = fp8 ? a.k_scales[l] : 1.f;
    pp.rope_vs[l] = fp8 ? a.v_scales[l] : 1.f;
    pp.attn_sl2[l] = a.attn.scale * kLog2e * (fp8 ? a.k_scales[l] : 1.f);
    pp.attn_vs[l] = fp8 ? a.v_scales[l] : 1.f;
  }
  pp.n_layers = a.n_layers;
  const int rows_per_block = [](int lpr) { return 256 / lpr; }(128);
  pp.nb_qkv = ceil_div(a.qkv.n_out, rows_per_block);
  pp.nb_o = ceil_div(a.o.n_out, rows_per_block);
  pp.nb_gu = ceil_div(a.gu.n_out, cfg_gu == 0 ? 256 / 32 : 256 / 64);
  pp.nb_down = ceil_div(a.down.n_out, 1);
  pp.nb_attn = a.plan.grid;
  pp.cfg_hidden = cfg_hidden;
  pp.cfg_gu = cfg_gu;
  pp.attn_nt = a.plan.nt;
  pp.barrier = a.barrier;
  int dev = 0, rate_khz = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && rate_khz > 0)
    pp.timeout_ticks = (unsigned long long)rate_khz * 250ull;  // 250 ms
  else
    pp.timeout_ticks = 25000000ull;  // 250 ms at 100 MHz
  const int grid = persistent_grid(a.attn.fp8);
  if (a.attn.fp8)
    hipLaunchKernelGGL(persist_kernel<true>, dim3(grid), dim3(256), 0, s, pp);
  else
    hipLaunchKernelGGL(persist_kernel<false>, dim3(grid), dim3(256), 0, s, pp);
  return hipGetLastError();
}

}  // namespace pkv
