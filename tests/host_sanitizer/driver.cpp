// Host-side driver for the sanitizer build of the POET library (AddressSanitizer and UndefinedBehaviorSanitizer on
// the host code only): every size and workspace query on valid and invalid sides and layers (the planning code that
// lays out workspaces), and the host validation of every entry point with arguments that it must reject before
// anything is launched. No GPU is needed: nothing here reaches a kernel launch. Exit status 0 when every call
// returned what it must; the sanitizers abort on the first memory or undefined-behavior error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "poet.h"

static int g_fail = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);     \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static void* const FAKE = reinterpret_cast<void*>(0x1000);  // never dereferenced: validation fails first

static poet_side side(int mode, int d, int b, int k, int dt) { return poet_side{mode, d, b, k, dt}; }

static poet_layer layer(int m, int n, int T, poet_side R, poet_side P, int act, int pad = 0) {
  poet_layer L;
  std::memset(&L, 0, sizeof(L));
  L.m = m; L.n = n; L.T = T; L.ldw = n + pad; L.ldx = n + pad; L.ldy = m + pad; L.act_dtype = act; L.R = R; L.P = P;
  return L;
}

int main() {
  EXPECT(std::strstr(poet_version(), "gfx950") != nullptr);
  for (int st = 0; st < 8; ++st) EXPECT(poet_status_string(st) != nullptr);
  EXPECT(std::strstr(poet_status_string(99), "unknown") != nullptr);
  EXPECT(std::strstr(poet_status_string(-1), "unknown") != nullptr);

  // sizes of valid and invalid sides
  const poet_side sides[] = {side(0, 2048, 256, 5, 1), side(0, 5461, 256, 5, 1), side(1, 5461, 2730, 5, 1),
                             side(1, 2048, 1024, 5, 1), side(0, 256, 32, 3, 0), side(0, 7, 7, 0, 0),
                             side(0, 10, 1, 2, 1), side(0, 300, 136, 4, 1), side(1, 1, 1, 1, 0)};
  for (const poet_side& s : sides) {
    EXPECT(poet_theta_len(&s) > 0 || s.b == 1);
    EXPECT(poet_num_prims(&s) > 0 && poet_prim_len(&s) > 0);
    (void)poet_powers_len(&s);
    (void)poet_build_workspace_bytes(&s, 0);
    (void)poet_build_workspace_bytes(&s, 1);
  }
  const poet_side bad[] = {side(2, 256, 32, 3, 0), side(0, 0, 32, 3, 0), side(0, 256, 0, 3, 0), side(0, 256, 300, 3, 0),
                           side(0, 256, 32, -1, 0), side(0, 256, 32, 17, 0), side(0, 256, 32, 3, 5),
                           side(1, 100, 101, 3, 0)};
  for (const poet_side& s : bad) {
    EXPECT(poet_theta_len(&s) == 0 && poet_prim_len(&s) == 0);
    EXPECT(std::strlen(poet_last_error()) > 0);
  }
  EXPECT(poet_theta_len(nullptr) == 0);
  EXPECT(poet_sample_workspace_bytes(5461) > 0 && poet_sample_workspace_bytes(0) == 0);

  // layer workspaces (every op), both paths, padded pitches, FS and BS
  std::vector<poet_layer> layers = {
      layer(2048, 2048, 16384, sides[0], sides[0], 1, 64), layer(5461, 2048, 16384, sides[1], sides[0], 1, 43),
      layer(2048, 5461, 16384, sides[0], sides[1], 1, 43), layer(5461, 2048, 4096, sides[2], sides[3], 1, 43),
      layer(256, 256, 64, sides[4], sides[4], 0), layer(300, 300, 0, sides[7], sides[7], 1, 4)};
  for (const poet_layer& L : layers) {
    for (int op = 0; op < 6; ++op) (void)poet_workspace_bytes(&L, op);
    EXPECT(poet_workspace_bytes(&L, 9) == 0);
    (void)poet_act_path_supported(&L);
  }
  std::vector<poet_side> all;
  for (const poet_layer& L : layers) { all.push_back(L.R); all.push_back(L.P); }
  EXPECT(poet_build_group_workspace_bytes((int)all.size(), all.data()) > 0);
  EXPECT(poet_adjoint_group_workspace_bytes((int)all.size(), all.data()) > 0);
  (void)poet_merge_group_workspace_bytes((int)layers.size(), layers.data());
  std::vector<poet_layer> act(layers.begin(), layers.begin() + 3);
  EXPECT(poet_fold_group_workspace_bytes((int)act.size(), act.data()) > 0);
  EXPECT(poet_spectral_workspace_bytes(5461, 2048) > 0);

  // host validation of every entry point: each call must be rejected before any launch
  const poet_layer L = layers[4];
  const size_t big = size_t(1) << 40;
  float* F = static_cast<float*>(FAKE);
  EXPECT(poet_build_orthogonal(&sides[4], F, nullptr, FAKE, nullptr, 0, FAKE, big, nullptr) == POET_E_ARG);
  EXPECT(poet_build_orthogonal(&sides[4], F, F, FAKE, nullptr, 7, FAKE, big, nullptr) == POET_E_ARG);
  EXPECT(poet_build_orthogonal(&bad[0], F, F, FAKE, nullptr, 0, FAKE, big, nullptr) != POET_OK);
  EXPECT(poet_build_orthogonal_exact(&sides[2], F, F, nullptr) == POET_E_UNSUPPORTED);
  EXPECT(poet_sample_indices(10, 11, 1, 2, 3, 4, static_cast<int32_t*>(FAKE), FAKE, big, nullptr) == POET_E_SHAPE);
  EXPECT(poet_sample_indices(100, 10, 1, 2, 3, 4, static_cast<int32_t*>(FAKE), FAKE, 4, nullptr) == POET_E_WORKSPACE);
  EXPECT(poet_sample_indices_noalloc(POET_NOALLOC_MAX_D + 1, 3, 1, 2, 3, 4, static_cast<int32_t*>(FAKE), nullptr) ==
         POET_E_SHAPE);
  EXPECT(poet_sample_permutation(0, 1, 2, 3, 4, static_cast<int32_t*>(FAKE), nullptr, nullptr) == POET_E_SHAPE);
  EXPECT(poet_gather2d(4, 4, 3, FAKE, 4, 4, 4, nullptr, nullptr, FAKE, 4, nullptr) == POET_E_ARG);
  EXPECT(poet_gather2d(5, 4, 2, FAKE, 4, 4, 4, nullptr, nullptr, FAKE, 4, nullptr) == POET_E_SHAPE);
  EXPECT(poet_linear_fwd(&L, nullptr, F, F, nullptr, nullptr, FAKE, FAKE, nullptr, FAKE, big, nullptr) == POET_E_ARG);
  EXPECT(poet_linear_fwd(&L, F, F, F, nullptr, nullptr, FAKE, FAKE, nullptr, FAKE, 16, nullptr) == POET_E_WORKSPACE);
  EXPECT(poet_linear_bwd(&L, F, F, F, nullptr, FAKE, nullptr, nullptr, nullptr, FAKE, FAKE, FAKE, F, F, FAKE, big,
                         nullptr) == POET_E_ARG);
  EXPECT(poet_linear_bwd_prims(&L, F, F, F, nullptr, nullptr, nullptr, FAKE, FAKE, FAKE, nullptr, F, FAKE, big,
                               nullptr) == POET_E_ARG);
  const poet_layer La = layers[0];
  const poet_layer Lf = layers[3];  // both sides FS in bf16
  int32_t* I = static_cast<int32_t*>(FAKE);
  EXPECT(poet_fs_form_workspace_bytes(&Lf) > 0);
  EXPECT(poet_fs_form(&La, F, F, F, nullptr, nullptr, FAKE, FAKE, FAKE, FAKE, big, nullptr) == POET_E_UNSUPPORTED);
  EXPECT(poet_fs_form(&Lf, F, F, F, I, I, FAKE, FAKE, FAKE, FAKE, 16, nullptr) == POET_E_WORKSPACE);
  EXPECT(poet_linear_fwd_formed(&Lf, nullptr, FAKE, FAKE, nullptr) == POET_E_ARG);
  EXPECT(poet_linear_bwd_formed_prims(&Lf, FAKE, nullptr, FAKE, I, I, FAKE, FAKE, FAKE, F, F, FAKE, big, nullptr) ==
         POET_E_ARG);
  EXPECT(poet_linear_bwd_formed_prims(&La, FAKE, FAKE, FAKE, nullptr, nullptr, FAKE, FAKE, FAKE, F, F, FAKE, big,
                                      nullptr) == POET_E_UNSUPPORTED);
  EXPECT(poet_weight_shadow(&La, nullptr, FAKE, nullptr) == POET_E_ARG);
  EXPECT(poet_linear_fwd_act(&L, FAKE, F, F, nullptr, nullptr, FAKE, FAKE, FAKE, FAKE, big, nullptr) != POET_OK);
  EXPECT(poet_linear_fwd_act(&La, FAKE, F, F, nullptr, nullptr, FAKE, FAKE, FAKE, FAKE, 16, nullptr) ==
         POET_E_WORKSPACE);
  EXPECT(poet_linear_bwd_act(&La, FAKE, F, F, nullptr, nullptr, nullptr, nullptr, FAKE, FAKE, FAKE, FAKE, F, F, FAKE,
                             big, nullptr) == POET_E_ARG);
  EXPECT(poet_linear_bwd_act_prims(&La, FAKE, F, F, nullptr, nullptr, FAKE, FAKE, FAKE, FAKE, nullptr, F, FAKE, big,
                                   nullptr) == POET_E_ARG);
  EXPECT(poet_linear_fwd_folded(&La, nullptr, F, nullptr, FAKE, FAKE, FAKE, FAKE, big, nullptr) == POET_E_ARG);
  EXPECT(poet_linear_bwd_folded_prims(&La, nullptr, F, nullptr, FAKE, FAKE, FAKE, FAKE, F, F, FAKE, big, nullptr) ==
         POET_E_ARG);
  std::vector<float*> tab(all.size(), F), nul(all.size(), nullptr);
  std::vector<void*> vtab(all.size(), FAKE);
  EXPECT(poet_build_orthogonal_group((int)all.size(), all.data(), const_cast<const float* const*>(tab.data()),
                                     tab.data(), nullptr, nullptr, 0, FAKE, big, nullptr) == POET_E_ARG);
  EXPECT(poet_build_orthogonal_group(-1, all.data(), nullptr, nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr) ==
         POET_E_ARG);
  EXPECT(poet_adjoint_group((int)all.size(), all.data(), const_cast<const float* const*>(tab.data()),
                            const_cast<const void* const*>(vtab.data()), nul.data(), FAKE, big, nullptr) ==
         POET_E_ARG);
  std::vector<void*> w0b(act.size(), nullptr);
  EXPECT(poet_fold_weights_group((int)act.size(), act.data(), const_cast<const void* const*>(w0b.data()), nullptr,
                                 nullptr, nullptr, nullptr, w0b.data(), nullptr, FAKE, big, nullptr) == POET_E_ARG);
  EXPECT(poet_merge(&L, F, nullptr, nullptr, F, F, F, nullptr, nullptr, 1, 2, 3, FAKE, big, nullptr) == POET_E_ARG);
  EXPECT(poet_merge_group(-1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                          nullptr, 1, nullptr, 0, nullptr) == POET_E_ARG);
  poet_adamw hp{1e-3f, 0.9f, 0.999f, 1e-8f, 0.f};
  poet_adamw hp_bad = hp;
  hp_bad.beta2 = 1.f;
  EXPECT(poet_adamw_group(2, all.data(), tab.data(), const_cast<const float* const*>(tab.data()), tab.data(),
                          tab.data(), &hp_bad, 1, nullptr) == POET_E_ARG);
  EXPECT(poet_adamw_group(2, all.data(), tab.data(), const_cast<const float* const*>(tab.data()), tab.data(),
                          tab.data(), &hp, 0, nullptr) == POET_E_ARG);
  EXPECT(poet_optimizer_reset_group(2, all.data(), nul.data(), tab.data(), nullptr) == POET_E_ARG);
  double* D = static_cast<double*>(FAKE);
  EXPECT(poet_hyperspherical_energy(64, 32, F, 16, 1.f, nullptr, D, FAKE, big, nullptr) == POET_E_SHAPE);
  EXPECT(poet_singular_value_entropy(64, 32, nullptr, 32, nullptr, D, FAKE, big, nullptr) == POET_E_ARG);
  EXPECT(poet_mfma_probe(0, 8, F, nullptr) == POET_E_ARG);
  EXPECT(poet_debug_gemm(nullptr, 0, nullptr, nullptr) == POET_E_ARG);
  int64_t n = 0;
  double ms = 0, fl = 0, by = 0;
  EXPECT(poet_profile_query(99, &n, &ms, &fl, &by) == POET_E_ARG);

  if (g_fail) std::fprintf(stderr, "%d checks failed\n", g_fail);
  else std::printf("host sanitizer driver: all checks passed\n");
  return g_fail ? 1 : 0;
}
