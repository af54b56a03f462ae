// Host-side checks of the C-ABI library under AddressSanitizer and UBSan.
//
// Built together with the library's host code only (no GPU code objects) by
// tests/test_host_sanitizers.py; every call here returns before a launch.
// Sweeps the pure size functions over normal and extreme shapes (their
// 64-bit size arithmetic and shape guards), and sends each entry point
// null, misaligned, mis-typed and mis-sized arguments, checking the status
// each one must return.  Exits non-zero on the first unexpected status;
// the sanitizers abort on any memory error or undefined behaviour.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "spectree.h"

namespace {

int failures = 0;

void expect(const char* what, long long got, long long want) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

// device-pointer stand-ins: never dereferenced on the host
alignas(256) unsigned char fake_mem[256];
void* const F = fake_mem;
void* const MIS = fake_mem + 4;                    // not 16-byte aligned

const int kShapes[][6] = {
    {8, 6, 32, 8, 128, 2054},      {64, 16, 64, 8, 128, 4112},   {16, 60, 64, 4, 128, 32828},
    {1, 1, 1, 1, 64, 1},           {1024, 64, 64, 1, 128, 64},   {1024, 6, 32, 8, 128, (1 << 21) - 1},
    {2, 64, 4, 2, 64, 200},        {3, 17, 48, 16, 64, 999},     {1, 64, 512, 8, 128, 1 << 20},
    // rejected: zero or negative sizes, N past 64, Hq not a multiple of Hkv,
    // unsupported D, S_max < N, products past 2^31
    {0, 6, 32, 8, 128, 2054},      {8, 0, 32, 8, 128, 2054},     {8, 65, 32, 8, 128, 2054},
    {8, 6, 30, 8, 128, 2054},      {8, 6, 32, 8, 96, 2054},      {8, 6, 32, 8, 128, 5},
    {-1, 6, 32, 8, 128, 2054},     {8, 6, 32, 0, 128, 2054},     {8, 6, 32, -8, 128, 2054},
    {1025, 6, 32, 8, 128, 2054},   {8, 6, 32, 8, 128, INT_MAX},  {INT_MAX, 64, 64, 1, 128, INT_MAX},
    {1024, 64, INT_MAX, 1, 128, 4096}, {4096, 64, 64, 64, 128, 1 << 20},
};

void sweep_sizes() {
  for (const auto& s : kShapes) {
    const size_t a = spec_tree_attn_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5]);
    const size_t a2 = spec_tree_attn_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5]);
    const size_t st = spec_verify_step_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5]);
    const size_t bw = spec_tree_attn_backward_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5]);
    expect("workspace bytes is a pure function", (long long)a, (long long)a2);
    // the step's workspace holds the attention's, after its own keys and counters
    if (a) expect("step workspace > attention workspace", st > a, 1);
    (void)bw;
  }
  // a sweep over many small shapes: every size function must return without UB
  for (int B = 1; B <= 9; B += 4)
    for (int N = 1; N <= 64; N += 7)
      for (int Hkv = 1; Hkv <= 8; Hkv *= 2)
        for (int g = 1; g <= 16; g *= 4)
          for (int D : {64, 128})
            for (int S : {N, N + 1, N + 63, N + 64, N + 4097}) {
              (void)spec_tree_attn_workspace_bytes(B, N, g * Hkv, Hkv, D, S);
              (void)spec_verify_step_workspace_bytes(B, N, g * Hkv, Hkv, D, S);
              (void)spec_tree_attn_backward_workspace_bytes(B, N, g * Hkv, Hkv, D, S);
            }
}

void entry_points() {
  const int B = 8, N = 6, Hq = 32, Hkv = 8, D = 128, S = 2054;
  const float sc = 0.088f;
  auto i32 = static_cast<const int32_t*>(F);
  auto u64 = static_cast<const uint64_t*>(F);
  auto f32 = static_cast<const float*>(F);
  const size_t ws = spec_tree_attn_workspace_bytes(B, N, Hq, Hkv, D, S);

  // mask build
  expect("mask null", spec_tree_mask_build(nullptr, B, N, (uint64_t*)F, nullptr, nullptr, nullptr), SPEC_ERR_NULL);
  expect("mask N=65", spec_tree_mask_build(i32, B, 65, (uint64_t*)F, nullptr, nullptr, nullptr), SPEC_ERR_SHAPE);
  expect("mask B=0", spec_tree_mask_build(i32, 0, N, (uint64_t*)F, nullptr, nullptr, nullptr), SPEC_ERR_SHAPE);

  // attention
  auto attn = [&](const void* q, spec_dtype qd, spec_dtype kd, int n, float s, void* w, size_t wb) {
    return spec_tree_attn_verify(q, qd, F, F, kd, f32, f32, i32, u64, B, n, Hq, Hkv, D, S, s, F, nullptr, w, wb,
                                 nullptr, nullptr);
  };
  expect("attn null q", attn(nullptr, SPEC_BF16, SPEC_BF16, N, sc, F, ws), SPEC_ERR_NULL);
  expect("attn dtype pair", attn(F, SPEC_F32, SPEC_BF16, N, sc, F, ws), SPEC_ERR_DTYPE);
  expect("attn q fp8", attn(F, SPEC_FP8_E4M3, SPEC_FP8_E4M3, N, sc, F, ws), SPEC_ERR_DTYPE);
  expect("attn unknown dtype", attn(F, static_cast<spec_dtype>(7), SPEC_BF16, N, sc, F, ws), SPEC_ERR_DTYPE);
  expect("attn negative dtype", attn(F, SPEC_BF16, static_cast<spec_dtype>(-1), N, sc, F, ws), SPEC_ERR_DTYPE);
  expect("attn N=65", attn(F, SPEC_BF16, SPEC_BF16, 65, sc, F, ws), SPEC_ERR_SHAPE);
  expect("attn scale<0", attn(F, SPEC_BF16, SPEC_BF16, N, -1.f, F, ws), SPEC_ERR_SHAPE);
  expect("attn scale nan", attn(F, SPEC_BF16, SPEC_BF16, N, __builtin_nanf(""), F, ws), SPEC_ERR_SHAPE);
  expect("attn misaligned q", attn(MIS, SPEC_BF16, SPEC_BF16, N, sc, F, ws), SPEC_ERR_ALIGN);
  expect("attn no workspace", attn(F, SPEC_BF16, SPEC_BF16, N, sc, nullptr, 0), SPEC_ERR_WORKSPACE);
  expect("attn short workspace", attn(F, SPEC_BF16, SPEC_BF16, N, sc, F, ws - 1), SPEC_ERR_WORKSPACE);
  expect("attn fp8 no scales",
         spec_tree_attn_verify(F, SPEC_BF16, F, F, SPEC_FP8_E4M3, nullptr, nullptr, i32, u64, B, N, Hq, Hkv, D, S,
                               sc, F, nullptr, F, ws, nullptr, nullptr),
         SPEC_ERR_NULL);

  // paged attention
  auto paged = [&](int ps, int np, int n) {
    return spec_tree_attn_verify_paged(F, SPEC_BF16, F, F, SPEC_BF16, nullptr, nullptr, i32, u64, i32, 129, ps, np,
                                       B, n, Hq, Hkv, D, sc, F, nullptr, nullptr, 0, nullptr, nullptr);
  };
  expect("paged page size 3", paged(3, 64, N), SPEC_ERR_SHAPE);
  expect("paged no pages", paged(16, 0, N), SPEC_ERR_SHAPE);
  expect("paged N=65", paged(16, 64, 65), SPEC_ERR_SHAPE);
  expect("paged no workspace", paged(16, 64, N), SPEC_ERR_WORKSPACE);

  // argmax and accept walk
  expect("argmax null", spec_vocab_argmax(nullptr, 4, 100, 100, (int32_t*)F, nullptr), SPEC_ERR_NULL);
  expect("argmax V=0", spec_vocab_argmax(f32, 4, 0, 100, (int32_t*)F, nullptr), SPEC_ERR_SHAPE);
  expect("argmax stride<V", spec_vocab_argmax(f32, 4, 100, 99, (int32_t*)F, nullptr), SPEC_ERR_SHAPE);
  int32_t* o = static_cast<int32_t*>(F);
  expect("walk null", spec_accept_walk(nullptr, u64, i32, i32, 1, N, 10, o, o, o, nullptr, nullptr), SPEC_ERR_NULL);
  expect("walk N=65", spec_accept_walk(i32, u64, i32, i32, 1, 65, 10, o, o, o, nullptr, nullptr), SPEC_ERR_SHAPE);
  expect("walk V=0", spec_accept_walk(i32, u64, i32, i32, 1, N, 0, o, o, o, nullptr, nullptr), SPEC_ERR_SHAPE);

  // commit
  expect("commit null", spec_commit_accepted(nullptr, F, SPEC_BF16, i32, i32, i32, B, N, Hkv, D, S, o, nullptr,
                                             nullptr, nullptr), SPEC_ERR_NULL);
  expect("commit fp4", spec_commit_accepted(F, F, SPEC_FP4_E2M1, i32, i32, i32, B, N, Hkv, D, S, o, nullptr, nullptr,
                                            nullptr), SPEC_ERR_DTYPE);
  expect("commit D=96", spec_commit_accepted(F, F, SPEC_BF16, i32, i32, i32, B, N, Hkv, 96, S, o, nullptr, nullptr,
                                             nullptr), SPEC_ERR_SHAPE);

  // fp8 / fp4 arithmetic
  expect("f8 null", spec_tree_attn_verify_f8(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 1, 1, 1,
                                             128, 8, 0.1f, nullptr, nullptr, nullptr, 0, nullptr, nullptr),
         SPEC_ERR_NULL);
  expect("f4 D=64", spec_tree_attn_verify_f4(F, F, F, f32, f32, i32, u64, B, N, Hq, Hkv, 64, S, sc, F, nullptr, F, ws,
                                             nullptr, nullptr), SPEC_ERR_SHAPE);

  // fp8 scores over a bf16 cache
  auto s8 = [&](const void* q, int d, void* w, size_t wb) {
    return spec_tree_attn_verify_f8_scores(q, F, F, nullptr, i32, u64, B, N, Hq, Hkv, d, S, sc, F, nullptr, w, wb,
                                           nullptr, nullptr);
  };
  expect("f8 scores null", s8(nullptr, D, F, ws), SPEC_ERR_NULL);
  expect("f8 scores D=64", s8(F, 64, F, ws), SPEC_ERR_SHAPE);
  expect("f8 scores misaligned", s8(MIS, D, F, ws), SPEC_ERR_ALIGN);
  expect("f8 scores short workspace", s8(F, D, F, ws - 1), SPEC_ERR_WORKSPACE);

  // backward
  const size_t bws = spec_tree_attn_backward_workspace_bytes(B, N, Hq, Hkv, D, S);
  auto bwd = [&](const void* q, spec_dtype dt, int n, void* w, size_t wb) {
    return spec_tree_attn_backward(q, F, F, dt, i32, u64, F, f32, F, B, n, Hq, Hkv, D, S, sc, F, F, F, w, wb, nullptr,
                                   nullptr);
  };
  expect("bwd null", bwd(nullptr, SPEC_BF16, N, F, bws), SPEC_ERR_NULL);
  expect("bwd fp8", bwd(F, SPEC_FP8_E4M3, N, F, bws), SPEC_ERR_DTYPE);
  expect("bwd unknown dtype", bwd(F, static_cast<spec_dtype>(99), N, F, bws), SPEC_ERR_DTYPE);
  expect("bwd N=65", bwd(F, SPEC_BF16, 65, F, bws), SPEC_ERR_SHAPE);
  expect("bwd misaligned", bwd(MIS, SPEC_BF16, N, F, bws), SPEC_ERR_ALIGN);
  expect("bwd no workspace", bwd(F, SPEC_BF16, N, nullptr, 0), SPEC_ERR_WORKSPACE);
  const size_t bwide = spec_tree_attn_backward_workspace_bytes(2, 60, 64, 4, 128, 460);
  expect("bwd wide short workspace",
         spec_tree_attn_backward(F, F, F, SPEC_BF16, i32, u64, F, f32, F, 2, 60, 64, 4, 128, 460, sc, F, F, F, F,
                                 bwide - 1, nullptr, nullptr),
         SPEC_ERR_WORKSPACE);

  // the one-launch step, with a workspace and with the static scratch
  const size_t sws = spec_verify_step_workspace_bytes(B, N, Hq, Hkv, D, S);
  auto step = [&](const void* q, int n, int64_t V, void* w, size_t wb) {
    return spec_verify_step(i32, i32, i32, q, SPEC_BF16, F, F, SPEC_BF16, nullptr, nullptr, f32, V, V, B, n, Hq, Hkv,
                            D, S, sc, (uint64_t*)F, nullptr, F, nullptr, o, o, o, o, w, wb, nullptr, nullptr);
  };
  expect("step null", step(nullptr, N, 1000, F, sws), SPEC_ERR_NULL);
  expect("step N=65", step(F, 65, 1000, F, sws), SPEC_ERR_SHAPE);
  expect("step V=0", step(F, N, 0, F, sws), SPEC_ERR_SHAPE);
  expect("step short workspace", step(F, N, 1000, F, sws - 1), SPEC_ERR_WORKSPACE);
  auto step_static = [&](int b, int n, int hq, int hkv, int s) {
    return spec_verify_step_static(i32, i32, i32, F, SPEC_BF16, F, F, SPEC_BF16, nullptr, nullptr, f32, 1000, 1000, b,
                                   n, hq, hkv, D, s, sc, (uint64_t*)F, nullptr, F, nullptr, o, o, o, o, nullptr,
                                   nullptr);
  };
  expect("static step too big", step_static(64, 60, 64, 4, 32828), SPEC_ERR_SCRATCH);
  expect("static step N=65", step_static(B, 65, Hq, Hkv, S), SPEC_ERR_SHAPE);

  // status strings
  for (int s = -5; s < 20; ++s) {
    const char* t = spec_status_string(s);
    expect("status string", t != nullptr && std::strlen(t) > 0, 1);
  }
}

}  // namespace

int main() {
  sweep_sizes();
  entry_points();
  if (failures) {
    std::fprintf(stderr, "%d host check(s) failed\n", failures);
    return 1;
  }
  std::printf("host checks OK\n");
  return 0;
}
