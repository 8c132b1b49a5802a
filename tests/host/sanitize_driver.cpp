// Host-side checks of the library's plain C++ part (chunk metadata, argument validation,
// workspace planning) under AddressSanitizer and UndefinedBehaviorSanitizer: random and
// adversarial inputs, each result checked against the invariants the header states.
// Built and run by tests/test_host_sanitizers.py; a sanitizer report fails that test.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>
#include <vector>

#include "ssd.h"
#include "ssd_plan.h"

static int g_fail = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond);   \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

// Invariants of the chunk metadata: every chunk inside one sequence, 1..cs tokens, ending
// at an absolute multiple of cs or at the sequence end, chunks maximal and in order.
static void check_metadata(int S, const std::vector<int32_t>& cu, const std::vector<int32_t>& nc,
                           int cs, int C, const std::vector<int32_t>& cuc,
                           const std::vector<int32_t>& sidx, const std::vector<int32_t>& last) {
  CHECK(cuc[0] == 0 && cuc[C] == cu[S]);
  int k = 0;
  for (int r = 0; r < S; ++r) {
    int t = cu[r];
    const int k0 = k;
    while (t < cu[r + 1]) {
      CHECK(k < C);
      if (k >= C) return;
      CHECK(sidx[k] == r && cuc[k] == t);
      const int64_t abs_start = int64_t(nc.empty() ? 0 : nc[r]) + (t - cu[r]);
      const int64_t to_boundary = cs - abs_start % cs;
      const int64_t len = std::min<int64_t>(to_boundary, cu[r + 1] - t);
      CHECK(cuc[k + 1] - cuc[k] == len);
      t += int(len);
      ++k;
    }
    CHECK(k > k0 && last[r] == k - 1);
  }
  CHECK(k == C);
}

static void metadata_random(std::mt19937& rng) {
  const int css[] = {1, 7, 16, 64, 256, 2048};
  for (int trial = 0; trial < 3000; ++trial) {
    const int S = int(rng() % 21);
    const int cs = css[rng() % 6];
    const bool with_nc = rng() % 2;
    std::vector<int32_t> cu(S + 1, 0), nc;
    for (int r = 0; r < S; ++r) cu[r + 1] = cu[r] + 1 + int(rng() % 700);
    if (with_nc) {
      nc.resize(S);
      for (auto& v : nc) v = int(rng() % 5000);
    }
    int32_t C = -1;
    const int32_t* ncp = with_nc ? nc.data() : nullptr;
    CHECK(ssd_chunk_metadata_count(S, cu.data(), ncp, cs, &C) == SSD_OK);
    if (C < 0) continue;
    std::vector<int32_t> cuc(C + 1), sidx(std::max(C, 1)), last(std::max(S, 1));
    int32_t got = -1;
    CHECK(ssd_build_chunk_metadata(S, cu.data(), ncp, cs, C, cuc.data(), sidx.data(), last.data(),
                                   &got) == SSD_OK);
    CHECK(got == C);
    check_metadata(S, cu, nc, cs, C, cuc, sidx, last);
    if (C > 0) {   // one short: capacity error with the required count, nothing else
      int32_t need = -1;
      CHECK(ssd_build_chunk_metadata(S, cu.data(), ncp, cs, C - 1, cuc.data(), sidx.data(),
                                     last.data(), &need) == SSD_ERR_CAPACITY);
      CHECK(need == C);
    }
  }
}

static void metadata_adversarial() {
  int32_t C = 0;
  std::vector<int32_t> cu = {0, 5, 9}, nc = {3, 0};
  std::vector<int32_t> cuc(16), sidx(16), last(16);
  CHECK(ssd_chunk_metadata_count(2, nullptr, nullptr, 4, &C) == SSD_ERR_NULL_POINTER);
  CHECK(ssd_chunk_metadata_count(2, cu.data(), nullptr, 4, nullptr) == SSD_ERR_NULL_POINTER);
  CHECK(ssd_chunk_metadata_count(-1, cu.data(), nullptr, 4, &C) == SSD_ERR_BAD_SHAPE);
  CHECK(ssd_chunk_metadata_count(2, cu.data(), nullptr, 0, &C) == SSD_ERR_BAD_SHAPE);
  CHECK(ssd_chunk_metadata_count(2, cu.data(), nullptr, -8, &C) == SSD_ERR_BAD_SHAPE);
  std::vector<int32_t> bad0 = {1, 5, 9};
  CHECK(ssd_chunk_metadata_count(2, bad0.data(), nullptr, 4, &C) == SSD_ERR_BAD_METADATA);
  std::vector<int32_t> empty = {0, 5, 5};   // a sequence with no new token
  CHECK(ssd_chunk_metadata_count(2, empty.data(), nullptr, 4, &C) == SSD_ERR_BAD_METADATA);
  std::vector<int32_t> down = {0, 5, 3};
  CHECK(ssd_chunk_metadata_count(2, down.data(), nullptr, 4, &C) == SSD_ERR_BAD_METADATA);
  std::vector<int32_t> negnc = {-1, 0};
  CHECK(ssd_chunk_metadata_count(2, cu.data(), negnc.data(), 4, &C) == SSD_ERR_BAD_METADATA);
  // positions near the int32 limit must be refused, not wrap
  const int32_t big = std::numeric_limits<int32_t>::max();
  std::vector<int32_t> cub = {0, big};
  std::vector<int32_t> ncb = {big};
  const ssd_status s = ssd_chunk_metadata_count(1, cub.data(), ncb.data(), 64, &C);
  CHECK(s == SSD_ERR_BAD_METADATA || s == SSD_ERR_BAD_SHAPE);
  CHECK(ssd_chunk_metadata_count(0, nullptr, nullptr, 4, &C) == SSD_OK && C == 0);
  int32_t got = -1;
  CHECK(ssd_build_chunk_metadata(2, cu.data(), nc.data(), 4, 16, cuc.data(), sidx.data(),
                                 last.data(), &got) == SSD_OK);
  CHECK(ssd_build_chunk_metadata(2, cu.data(), nc.data(), 4, 16, nullptr, sidx.data(),
                                 last.data(), &got) == SSD_ERR_NULL_POINTER);
}

// Every (dtype, P, N, cs, a_kind, mode) combination, valid or not: the plan either refuses
// with a status or returns a workspace whose parts lie inside it.
static void plan_sweep() {
  static int fake[64];
  void* F = fake;
  const int Ps[] = {1, 16, 32, 64, 128}, Ns[] = {16, 32, 64, 128, 256}, css[] = {24, 64, 128, 256, 512};
  int ok = 0;
  for (int dtype : {int(SSD_F32), int(SSD_BF16), 7})
    for (int P : Ps)
      for (int N : Ns)
        for (int cs : css)
          for (int kind : {int(SSD_A_SCALAR), int(SSD_A_DIAG)})
            for (int bs : {0, 2 * cs, cs + 1}) {
              ssd_prefill_args a{};
              a.T = 4096; a.H = kind == SSD_A_DIAG ? 200 : 8; a.P = P; a.G = kind == SSD_A_DIAG ? 1 : 2;
              a.N = N; a.chunk_size = cs; a.num_seqs = 3; a.num_chunks = 3 + 4096 / cs;
              a.in_dtype = dtype; a.a_kind = kind;
              a.x = a.dt = a.B = a.C = F; a.y = F; a.A = reinterpret_cast<const float*>(F);
              a.x_stride_t = a.y_stride_t = int64_t(a.H) * P; a.dt_stride_t = a.H;
              a.bc_stride_t = int64_t(a.G) * N;
              a.cu_seqlens = a.cu_chunk_seqlens = a.seq_idx = a.last_chunk_indices =
                  reinterpret_cast<const int32_t*>(F);
              a.dt_min = 0.f; a.dt_max = std::numeric_limits<float>::infinity();
              a.block_size = bs;
              if (bs) {
                a.idx_stride = 8; a.num_computed = reinterpret_cast<const int32_t*>(F);
                a.state_pool = F; a.state_indices = reinterpret_cast<const int32_t*>(F);
                a.num_slots = 16; a.slot_stride = int64_t(a.H) * P * N;
              }
              ssd::PrefillPlan plan;
              const ssd_status st = ssd::plan_prefill(&a, &plan);
              CHECK(st >= SSD_OK && st <= SSD_ERR_HIP);
              if (st == SSD_OK) {
                ++ok;
                const size_t offs[] = {plan.off_cb, plan.off_bt, plan.off_dc, plan.off_cf,
                                       plan.off_ord, plan.off_flag, plan.off_items, plan.off_ring,
                                       plan.off_blk};
                for (size_t o : offs) CHECK(o <= plan.ws_bytes);
                CHECK(plan.ws_bytes % 256 == 0);
              }
            }
  CHECK(ok > 10);
  CHECK(ssd::plan_prefill(nullptr, nullptr) != SSD_OK);
}

static void decode_sweep() {
  static int fake[64];
  void* F = fake;
  for (int N : {8, 16, 32, 64, 128, 256, 512})
    for (int ntok : {0, 1, 4, 16, 17})
      for (int kind : {int(SSD_A_SCALAR), int(SSD_A_DIAG), 3}) {
        ssd_decode_args a{};
        a.B_pad = 512; a.ntok = ntok; a.H = kind == SSD_A_SCALAR ? 48 : 256;
        a.P = kind == SSD_A_SCALAR ? 64 : 1; a.G = kind == SSD_A_SCALAR ? 4 : 1; a.N = N;
        a.in_dtype = SSD_BF16; a.a_kind = kind;
        a.x = a.dt = a.B = a.C = F; a.y = F; a.A = reinterpret_cast<const float*>(F);
        a.state_pool = F; a.slot_stride = int64_t(a.H) * a.P * N; a.num_slots = 2048;
        a.state_indices = reinterpret_cast<const int32_t*>(F);
        a.dt_min = 0.f; a.dt_max = 1e30f;
        const ssd_status st = ssd::check_decode(&a);
        CHECK(st >= SSD_OK && st <= SSD_ERR_HIP);
      }
  CHECK(ssd::check_decode(nullptr) != SSD_OK);
}

int main() {
  std::mt19937 rng(12345);
  metadata_random(rng);
  metadata_adversarial();
  plan_sweep();
  decode_sweep();
  for (int s = -1; s <= 9; ++s) CHECK(ssd_status_string(static_cast<ssd_status>(s)) != nullptr);
  CHECK(ssd_abi_version() > 0);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
