// ssd_entry.hip -- C-ABI entry points that launch kernels: argument resolution, the
// device-facing checks (alignment of vector accesses, workspace), and the launch sequence.
#include <atomic>
#include <cstdint>

#include "ssd_params.h"

// The workspace of ssd_prefill_noalloc: one copy per GPU, in the code object's device
// memory, shared by every such call on that GPU (see include/ssd.h).
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of this GPU's `scratch` (the host-side name is only a stand-in), looked
// up once per device with that device current and kept; NULL if the lookup failed.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    // racing first calls on one device both find the same address
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// The chunked kernels read x, B, C rows and write y rows with 16-byte vector accesses and
// move states as float4: check the pointers and strides allow that.
ssd_status check_vector_access(const ssd_prefill_args* a) {
  const int esz = a->in_dtype == SSD_BF16 ? 2 : 4;
  const int64_t per16 = 16 / esz;
  if (!aligned(a->x, 16) || !aligned(a->B, 16) || !aligned(a->C, 16) || !aligned(a->y, 16))
    return SSD_ERR_UNSUPPORTED;
  if (a->x_stride_t % per16 || a->bc_stride_t % per16 || a->y_stride_t % per16)
    return SSD_ERR_UNSUPPORTED;
  if (a->state_pool && (!aligned(a->state_pool, 16) || a->slot_stride % 4))
    return SSD_ERR_UNSUPPORTED;
  if (a->chunk_states_out && !aligned(a->chunk_states_out, 16)) return SSD_ERR_UNSUPPORTED;
  if (a->chunk_local_states_out && !aligned(a->chunk_local_states_out, 16))
    return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

}  // namespace

extern "C" {

ssd_status ssd_prefill_workspace_size(const ssd_prefill_args* a, size_t* bytes) {
  if (!bytes) return SSD_ERR_NULL_POINTER;
  ssd::PrefillPlan plan;
  const ssd_status st = ssd::plan_prefill(a, &plan);
  if (st != SSD_OK) return st;
  *bytes = plan.ws_bytes;
  return SSD_OK;
}

}  // extern "C"

namespace {

// ssd_prefill after planning and the workspace check: the device-facing checks, argument
// resolution and the launches.
ssd_status prefill_launch(const ssd_prefill_args* a, const ssd::PrefillPlan& plan, void* workspace,
                          ssd_stream_t stream) {
  ssd_status st = SSD_OK;
  if (plan.kind == ssd::PrefillKind::kChunked) {
    st = check_vector_access(a);
    if (st != SSD_OK) return st;
  } else if (a->state_pool && (!aligned(a->state_pool, 16) || a->slot_stride % 4)) {
    return SSD_ERR_UNSUPPORTED;
  } else if (a->chunk_states_out && !aligned(a->chunk_states_out, 16)) {
    return SSD_ERR_UNSUPPORTED;
  }

  ssd::PrefillParams p{};
  p.T = a->T; p.H = a->H; p.P = a->P; p.G = a->G; p.N = a->N;
  p.S = a->num_seqs; p.C = a->num_chunks; p.cs = a->chunk_size;
  p.x = a->x; p.x_st = a->x_stride_t;
  p.dt = a->dt; p.dt_st = a->dt_stride_t;
  p.B = a->B; p.Cm = a->C; p.bc_st = a->bc_stride_t;
  p.y = a->y; p.y_st = a->y_stride_t;
  p.A = a->A; p.D = a->D;
  p.prep = ssd::DtPrep{a->dt_bias, a->dt_softplus ? 1 : 0, a->dt_min, a->dt_max};
  p.cu_seqlens = a->cu_seqlens; p.cu_chunk = a->cu_chunk_seqlens;
  p.seq_idx = a->seq_idx; p.last_chunk = a->last_chunk_indices;
  p.pool = a->state_pool; p.slot_stride = a->slot_stride; p.num_slots = a->num_slots;
  p.pool_kind = a->state_dtype;
  p.state_idx = a->state_indices; p.has_init = a->has_initial_state;
  p.write_final = (a->write_final_to_pool && a->state_pool) ? 1 : 0;
  p.block_size = a->block_size; p.idx_stride = a->block_size > 0 ? a->idx_stride : 1;
  p.num_computed = a->num_computed;
  p.blk_last_comp = a->block_idx_last_computed; p.blk_last_sched = a->block_idx_last_scheduled;
  p.flag = a->device_error_flag;
  p.dA_cumsum_out = a->dA_cumsum_out;
  p.cb_out = a->cb_out;
  p.local_states_out = a->chunk_local_states_out;
  char* ws = static_cast<char*>(workspace);
  p.states = a->chunk_states_out;
  if (plan.kind == ssd::PrefillKind::kChunked) {
    p.cbw = ws + plan.off_cb;
    p.btw = ws + plan.off_bt;
    p.dcw = plan.chain ? nullptr : reinterpret_cast<float*>(ws + plan.off_dc);
    p.cfw = ws + plan.off_cf;
    p.seq_ord = reinterpret_cast<int*>(ws + plan.off_ord);
    p.blk_slot = a->block_size > 0 ? reinterpret_cast<int*>(ws + plan.off_blk) : nullptr;
    if (plan.chain) {
      p.chain_flag = reinterpret_cast<int*>(ws + plan.off_flag);
      p.items = plan.off_items ? reinterpret_cast<int*>(ws + plan.off_items) : nullptr;
      p.chain_grid = plan.chain_grid;
      p.hring = a->chunk_states_out ? nullptr : reinterpret_cast<float*>(ws + plan.off_ring);
    }
  }

  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (ssd::debug_checks_enabled() && ssd::launch_prefill_slot_check(p, s) != hipSuccess)
    return SSD_ERR_HIP;
  const hipError_t e = plan.kind == ssd::PrefillKind::kChunked
                           ? ssd::launch_chunked_prefill(plan.variant, p, s, a->profile_events)
                           : ssd::launch_diag_prefill(a->in_dtype, a->a_kind == SSD_A_SCALAR, p,
                                                      s, a->profile_events);
  return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

extern "C" {

ssd_status ssd_prefill(const ssd_prefill_args* a, void* workspace, size_t workspace_bytes,
                       ssd_stream_t stream) {
  ssd::PrefillPlan plan;
  const ssd_status st = ssd::plan_prefill(a, &plan);
  if (st != SSD_OK) return st;
  if (a->num_seqs == 0) return SSD_OK;
  if (plan.ws_bytes > 0 &&
      (!workspace || workspace_bytes < plan.ws_bytes || !aligned(workspace, 256)))
    return SSD_ERR_WORKSPACE;
  return prefill_launch(a, plan, workspace, stream);
}

ssd_status ssd_prefill_noalloc(const ssd_prefill_args* a, ssd_stream_t stream) {
  ssd::PrefillPlan plan;
  const ssd_status st = ssd::plan_prefill(a, &plan);
  if (st != SSD_OK) return st;
  if (a->num_seqs == 0) return SSD_OK;
  if (plan.ws_bytes > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    ws = scratch_ptr();
    if (!ws) return SSD_ERR_HIP;
  }
  return prefill_launch(a, plan, ws, stream);
}

ssd_status ssd_prefill_kernel_count(const ssd_prefill_args* a, int32_t* count,
                                    const char** names) {
  if (!count) return SSD_ERR_NULL_POINTER;
  ssd::PrefillPlan plan;
  const ssd_status st = ssd::plan_prefill(a, &plan);
  if (st != SSD_OK) return st;
  static const char* const kChunked[] = {"k_chunk_prep", "k_chunk_march"};
  static const char* const kChain[] = {"k_chunk_prep", "k_chunk_chain"};
  static const char* const kDiag[] = {"k_diag_scan"};
  static const char* const kDiagMixed[] = {"k_diag_scan_mixed"};
  *count = 0;
  if (a->num_seqs == 0) return SSD_OK;
  const char* const* list =
      plan.kind == ssd::PrefillKind::kChunked ? (plan.chain ? kChain : kChunked)
      : ssd::diag_mixed_grid(a->a_kind == SSD_A_SCALAR, a->num_seqs, a->H, a->G, a->N)
          ? kDiagMixed : kDiag;
  *count = plan.kind == ssd::PrefillKind::kChunked ? 2 : 1;
  if (names)
    for (int i = 0; i < *count; ++i) names[i] = list[i];
  return SSD_OK;
}

ssd_status ssd_state_update(const ssd_decode_args* a, ssd_stream_t stream) {
  ssd_status st = ssd::check_decode(a);
  if (st != SSD_OK) return st;
  if (a->B_pad == 0) return SSD_OK;
  if (ssd::decode_lds_bytes(a->ntok, a->P, a->N) > 64 * 1024) return SSD_ERR_UNSUPPORTED;
  if (!aligned(a->state_pool, 16) || a->slot_stride % 4) return SSD_ERR_UNSUPPORTED;
  // A 2-byte pool (bf16, fp16) is moved 8 states (16 bytes) per lane by the dense-A kernel.
  if (a->state_dtype != SSD_F32 && a->a_kind == SSD_A_SCALAR && a->slot_stride % 8)
    return SSD_ERR_UNSUPPORTED;
  ssd::DecodeParams p{};
  p.B_pad = a->B_pad; p.ntok = a->ntok; p.H = a->H; p.P = a->P; p.G = a->G; p.N = a->N;
  p.diag = a->a_kind == SSD_A_DIAG ? 1 : 0;
  p.x = a->x; p.dt = a->dt; p.B = a->B; p.Cm = a->C; p.y = a->y;
  p.A = a->A; p.D = a->D;
  p.prep = ssd::DtPrep{a->dt_bias, a->dt_softplus ? 1 : 0, a->dt_min, a->dt_max};
  p.pool = a->state_pool; p.slot_stride = a->slot_stride; p.num_slots = a->num_slots;
  p.pool_kind = a->state_dtype;
  p.idx = a->state_indices; p.num_acc = a->num_accepted_tokens;
  p.null_id = a->null_block_id; p.flag = a->device_error_flag;
  p.idx_stride = a->idx_stride;
  p.blk_last_comp = a->block_idx_last_computed; p.blk_last_sched = a->block_idx_last_scheduled;
  if (ssd::debug_checks_enabled() &&
      ssd::launch_decode_slot_check(p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSD_ERR_HIP;
  const hipError_t e = ssd::launch_state_update(a->in_dtype, p, static_cast<hipStream_t>(stream),
                                                a->profile_events);
  return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
