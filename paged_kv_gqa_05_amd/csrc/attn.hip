// Paged GQA decode attention for gfx950: split over the context, with the
// merge of a row's partitions done by the last of them to finish.
//
// What it computes (rvLLM post on discuss.pytorch.kr, section
// "PagedAttention과 FlashAttention-3": block-table KV cache, GQA reads each KV
// head once for its whole group of query heads, f16 KV or FP8 E4M3 KV):
//   out[b][h] = sum_t softmax_t(scale * <q[b][h], K_t>) V_t,  t < context_lens[b]
// with K_t, V_t gathered through the row's block table.
//
// Design (MI355X, not the pages' FlashAttention-3 kernels):
//  * One workgroup of W waves (4 or 8) per (row b, KV head g, partition of
//    16 NT W tokens), partition-major: blockIdx = partition * B * Hkv +
//    b * Hkv + g, so that every row's first partition is dispatched before
//    any later one; partitions beyond a row's context exit at once.  The row's block-table entries and
//    the query rows are loaded together with the context length, so a
//    workgroup waits one memory round trip before its KV loads.
//  * Wave w of a partition owns its blocks w, w + W, ... (at most NT) and loads
//    all of their K and V at once.  K blocks are stored in 16-byte chunks of
//    8 dims x 16 tokens (fp8: 16 dims).  f16 V blocks are dim-major [D][16]
//    (one 16-byte load gives a lane 8 tokens of one dim); fp8 V blocks are
//    [D/64][4][16][4][4] (dim group, token quad, dim in group, dim step of
//    16, token in quad), so one 16-byte load gives a lane its four
//    token-quad fragments of dims n, n + 16, n + 32, n + 48 and a wave
//    instruction reads 1 KB (1.16x faster than 4-byte loads at the long
//    fp8 workload).
//  * Scores: K rows feed v_mfma_f32_16x16x32_f16 from registers as the A
//    operand (token = MFMA row), the group's query rows (G <= 16, zero padded)
//    are the B operand, giving S^T [token][head].  The dot product over D is
//    taken in a permuted dim order (the same for q and K), which is what makes
//    the K loads contiguous.  f16 takes the wave's blocks in pairs and gives
//    the two score products of a pair their K rows in a permuted token order,
//    so that each lane's accumulators hold 8 consecutive tokens of one block:
//    exactly the B operand of v_mfma_f32_16x16x32_f16 for O^T += V^T P^T,
//    whose A operand is one 16-byte V load per lane (64 tile loads for a wave
//    of 8 blocks, against 96 with 8-byte V loads and the 16x16x16 product).
//    fp8 keeps one block per product: its accumulators are the B operand of
//    v_mfma_f32_16x16x16f16, whose A operand comes from the V block's codes.
//    No LDS and no shuffles between the two products either way.
//  * Softmax per wave in two passes over registers: all scores first, one max
//    per head, then P = exp2(S - max) and the PV products with no rescaling
//    (an online softmax rescales the 32 output accumulators at every block,
//    which cost more than the loads).  The W waves' (max, sum, O) are
//    combined through LDS.
//  * A row with a single partition writes its normalised f16 output directly.
//    Otherwise each partition stores (max, sum, unnormalised O) in fp32 with
//    device-coherent stores and counts its arrival on a per-(row, KV head)
//    counter; the workgroup that arrives last merges all partitions of the
//    row in partition order (so the result does not depend on arrival order),
//    writes the output and resets the counter to zero.  When the whole grid
//    is resident at once (8-wave plans), the row's first partition instead
//    keeps its own partial on chip, waits for the others' arrivals and
//    merges (falling back to publishing after a bounded wait).  One kernel, no merge
//    launch; the counters are zero before and after every call.
//  * FP8 E4M3 codes are converted to f16 in registers with the gfx950
//    conversion instruction (exact: every E4M3 value is an f16 value); the
//    per-tensor K scale is folded into the score scale and the V scale into
//    the output.
#include <algorithm>

#include "attn_body.h"

namespace pkv {
namespace {

template <int D, bool FP8, int NT, int kWaves>
__global__ void __launch_bounds__(64 * kWaves, (attn_min_waves<NT, kWaves>())) attn_kernel(SplitParams p) {
  attn_body<D, FP8, NT, kWaves, false>(p, blockIdx.x);
}

// The work-list form (4 waves), a kernel of its own: its item loop needs more
// registers than the direct form, whose residency must not change.
template <int D, bool FP8, int NT, int W>
__global__ void __launch_bounds__(64 * W) attn_wl_kernel(SplitParams p) {
  attn_worklist<D, FP8, NT, W>(p);
}

// Workgroups of one configuration that the device holds at once (occupancy
// query, cached per device).
template <int D, bool FP8, int NT, int W>
int resident_workgroups() {
  static int cache[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_wl_kernel<D, FP8, NT, W>, 64 * W, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = per_cu * cus > 0 ? per_cu * cus : -1;
  }
  return cache[dev];
}

template <int D, bool FP8, int NT, int W>
void launch_cfg(const SplitParams& sp, const AttnPlan& plan, hipStream_t s) {
  hipLaunchKernelGGL((attn_kernel<D, FP8, NT, W>), dim3(plan.grid), dim3(64 * W), 0, s, sp);
}

// The work-list form: as many workgroups as the device holds at once (any
// other count gives the same result).
template <int D, bool FP8, int W>
void launch_worklist(SplitParams sp, const AttnPlan& plan, hipStream_t s) {
  sp.worklist = 1;
  const int resident = resident_workgroups<D, FP8, 8, W>();
  const int grid = resident > 0 ? std::min(resident, plan.grid) : plan.grid;
  hipLaunchKernelGGL((attn_wl_kernel<D, FP8, 8, W>), dim3(grid), dim3(64 * W), 0, s, sp);
}

template <int D, bool FP8>
hipError_t launch_impl(const SplitParams& sp, const AttnPlan& plan, hipStream_t s) {
  if (plan.worklist && attn_worklist_enabled) {
    if constexpr (FP8) {
      if (plan.waves == 8) {
        launch_worklist<D, FP8, 8>(sp, plan, s);
        return hipGetLastError();
      }
    }
    launch_worklist<D, FP8, 4>(sp, plan, s);
    return hipGetLastError();
  }
  if (plan.waves == 8) {
    if constexpr (!FP8) {
      if (plan.nt == 6) {
        launch_cfg<D, FP8, 6, 8>(sp, plan, s);
        return hipGetLastError();
      }
    }
    launch_cfg<D, FP8, 8, 8>(sp, plan, s);
  } else {
    switch (plan.nt) {
      case 2: launch_cfg<D, FP8, 2, 4>(sp, plan, s); break;
      case 4: launch_cfg<D, FP8, 4, 4>(sp, plan, s); break;
      default: launch_cfg<D, FP8, 8, 4>(sp, plan, s); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

unsigned long long attn_merge_wait_ticks = 10000;  // 100 us at the 100 MHz wall clock
int attn_worklist_enabled = 1;

AttnPlan attn_plan(int batch, int hq, int hkv, int head_dim, int elt_bytes, int max_context) {
  AttnPlan p{};
  // A workgroup of W waves takes one partition of 16 NT W tokens; every wave
  // holds the K and V of its NT blocks in registers (NT = 8 at most).
  // Partitions of one row are merged through memory (coherent stores, an
  // arrival atomic and a re-read by the last one), which lengthens the
  // critical path, so partitions are as large as possible while every
  // workgroup of the call can still be resident at once:
  //  * 8 waves x 8 blocks (1024 tokens, one workgroup per CU) when a row can
  //    exceed 512 tokens and the partitions fit in 256 workgroups, unless
  //    that is one partition per row for fewer than 192 rows (then 4 x 4);
  //  * with more rows of at most 768 f16 tokens, 8 waves x 6 blocks (one
  //    partition per row over two rounds);
  //  * else 4 waves x 8 blocks (512 tokens, one per CU: 296 registers at f16);
  //  * else, when those exceed 256 workgroups, 4 waves x 4 blocks (256
  //    tokens, three per CU) if that fits in 768;
  //  * calls that need several rounds anyway keep 4 x 8 (measured best on the
  //    long fp8 workload);
  //  * rows short enough for one 4-wave partition take no more blocks per
  //    wave than they need (at least 4).
  // Fewer blocks per wave also when the grid would hold fewer workgroups than
  // CUs.  The estimate uses max_context for every row.
  const int mc = max_context > 0 ? max_context : 1;
  const long rows = (long)batch * hkv;
  auto wgs = [&](int w, int nt) { return rows * ceil_div(mc, 16 * nt * w); };
  int waves = 4, nt = 8;
  // (at most 16 rows: 4-wave partitions, which the persistent batch-1 step
  // also runs; 8-wave ones would leave it)
  if (mc > 512 && mc <= 1024 && rows > 16 && rows < 192) {
    // one 8-wave partition per row would leave a quarter or more of the CUs
    // idle: 256-token partitions instead (7B heads, batch 32, contexts
    // 512-545, 128 rows: 12.2-13.1 -> 12.0-12.2 us)
    nt = 4;
  } else if (mc > 512 && wgs(8, 8) <= 256 && rows > 16) {
    waves = 8;
  } else if (elt_bytes == 2 && mc > 512 && mc <= 768 && rows > 256) {
    // more than 256 rows of at most 768 tokens: one 8-wave partition of 6
    // blocks a wave per row, so no row is split into a full partition and a
    // few-token remainder with its merge (7B heads at batch 128, contexts
    // 512-545, 512 rows: 40.9-41.8 -> 30.1-30.8 us; 8 x 8 blocks 31.7-32.5)
    waves = 8;
    nt = 6;
  } else {
    if (wgs(4, 8) > 256 && wgs(4, 4) <= 768) nt = 4;
    while (nt > 2 && wgs(4, nt) < 256 && ceil_div(mc, 64 * nt) > 1) nt /= 2;
    // short rows: no more blocks per wave than a row can give each of the 4
    // waves (a wave issues the loads of all nt blocks; at 165 tokens, 4 and
    // not 8: decode step at batch 1 1.072 -> 1.027 ms, batch 64 1.887 -> 1.840 ms)
    const int per_wave = ceil_div(ceil_div(mc, 16), 4);
    while (nt > 4 && per_wave <= nt / 2) nt /= 2;
  }
  // Long rows (8 or more 512-token partitions at max_context) over a grid of
  // several rounds: the work-list form (attn_worklist), with 1024-token items
  // for fp8 (8 waves x 8 blocks; f16 would spill at that size).  fp8long
  // (32 rows x 4 KV heads, contexts 1106..30229): 103.3-103.6 us direct,
  // 100.9 with 512-token items, 96.6-96.9 with 1024-token items.  Calls of a
  // few partitions per row keep the direct grid (7B heads, batch 128,
  // contexts 512-540: 47.0 us either way).
  int worklist = 0;
  if (batch <= kWorklistMaxRows && rows > 16 && waves == 4 && nt == 8 && ceil_div(mc, 512) >= 8 &&
      wgs(4, 8) > 512) {
    worklist = 1;
    if (elt_bytes == 1) waves = 8;
  }
  p.worklist = worklist;
  p.waves = waves;
  p.nt = nt;
  p.max_context = mc;
  p.part = 16 * nt * waves;
  p.n_parts_max = ceil_div(mc, p.part);
  p.grid = batch * hkv * p.n_parts_max;
  // (the work-list form's item counter and exit count follow the arrival counters)
  p.counter_bytes = align_up(((size_t)batch * hkv + 2) * sizeof(int), 256);
  const size_t ml = align_up((size_t)batch * hq * p.n_parts_max * sizeof(float2), 256);
  const size_t o = align_up((size_t)batch * hq * p.n_parts_max * head_dim * sizeof(float), 256);
  p.ws_bytes = p.counter_bytes + (p.n_parts_max > 1 ? ml + o : 0);
  return p;
}

hipError_t launch_paged_attention(const AttnArgs& a, const AttnPlan& plan, hipStream_t s) {
  const SplitParams sp = make_split_params(a, plan);
  if (a.head_dim == 128) return a.fp8 ? launch_impl<128, true>(sp, plan, s) : launch_impl<128, false>(sp, plan, s);
  return a.fp8 ? launch_impl<64, true>(sp, plan, s) : launch_impl<64, false>(sp, plan, s);
}

}  // namespace pkv

#ifdef PKV_ATTN_STAMPS
extern "C" int pkv_debug_attn_stamps(void* host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(pkv::g_attn_stamps), bytes, 0, hipMemcpyDeviceToHost);
}
extern "C" int pkv_debug_attn_stamps_clear(const void* zeros, size_t bytes) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(pkv::g_attn_stamps), zeros, bytes, 0, hipMemcpyHostToDevice);
}
#endif

extern "C" pkv_status pkv_debug_attn_worklist(int enable) {
  pkv::attn_worklist_enabled = enable;
  return PKV_OK;
}

extern "C" pkv_status pkv_debug_attn_merge_wait(unsigned long long ticks) {
  pkv::attn_merge_wait_ticks = ticks;
  return PKV_OK;
}
