// Driver of the C ABI's host-side argument checks for a sanitizer build (address and
// undefined behaviour).  Every call here fails validation before any device work, so it
// runs without a GPU; each must return its status code and leave a message.
#include <stdio.h>
#include <string.h>

#include "../../include/dg.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static dg_model_cfg base_cfg() {
    dg_model_cfg c;
    memset(&c, 0, sizeof(c));
    c.n_layers = 2; c.d_model = 256; c.n_q_heads = 4; c.n_kv_heads = 2; c.head_dim = 64;
    c.n_experts = 8; c.top_k = 2; c.d_ff = 512; c.vocab = 1024; c.canvas = 256; c.max_ctx = 320;
    c.rope_base = 10000.0; c.rms_eps = 1e-6f; c.temperature = 1.0f;
    c.act_dtype = DG_F32; c.expert_dtype = DG_F32;
    return c;
}

int main() {
    dg_handle* h = nullptr;
    CHECK(dg_create(nullptr, &h) == DG_EINVAL && h == nullptr);
    CHECK(dg_create(nullptr, nullptr) == DG_EINVAL);
    const int n_bad = 11;
    for (int i = 0; i < n_bad; ++i) {
        dg_model_cfg c = base_cfg();
        switch (i) {
            case 0: c.n_layers = 0; break;
            case 1: c.n_q_heads = 3; break;
            case 2: c.top_k = 9; break;
            case 3: c.canvas = 2048; break;
            case 4: c.max_ctx = 100; break;
            case 5: c.temperature = 0.0f; break;
            case 6: c.act_dtype = 7; break;
            case 7: c.act_dtype = DG_BF16; c.expert_dtype = DG_BF16; c.head_dim = 64; break;
            case 8: c.n_experts = 300; break;
            case 9: c.max_batch = -1; break;
            case 10: c.max_batch = 257; break;
        }
        CHECK(dg_create(&c, &h) == DG_EINVAL);
        CHECK(strlen(dg_last_error()) > 0);
    }
    CHECK(dg_denoise_step(nullptr, nullptr, nullptr, 0, 12, 0, nullptr) == DG_EINVAL);
    CHECK(dg_generate_block(nullptr, nullptr, 12, 0, 1, nullptr) == DG_EINVAL);
    CHECK(dg_prefill_prompt_kv(nullptr, nullptr, 0, nullptr) == DG_EINVAL);
    CHECK(dg_commit_canvas(nullptr, nullptr, nullptr) == DG_EINVAL);
    CHECK(dg_get_state(nullptr, nullptr, nullptr) == DG_EINVAL);
    dg_destroy(nullptr);
    size_t ws = 0;
    CHECK(dg_attention_workspace_size(16, 8, 256, 4352, 128, 0, 0, DG_BF16, &ws) == DG_OK);
    CHECK(ws == (size_t)8 * 128 * 4352 * 2 + (size_t)16 * 16 * 256 * (128 * 2 + 8));
    CHECK(dg_attention_workspace_size(16, 8, 256, 4352, 64, 0, 0, DG_BF16, &ws) == DG_EINVAL);
    CHECK(dg_attention_workspace_size(16, 8, 256, 4352, 128, 0, 0, DG_BF16, nullptr) == DG_EINVAL);
    CHECK(dg_attention_workspace_size(16, 7, 256, 4352, 128, 0, 0, DG_BF16, &ws) == DG_EINVAL);
    char dummy[64];
    CHECK(dg_attention(nullptr, dummy, dummy, dummy, 16, 8, 256, 4352, 128, 0.1f, 0, 0, DG_BF16,
                       dummy, sizeof(dummy), nullptr) == DG_EINVAL);
    CHECK(dg_attention(dummy, dummy, dummy, dummy, 16, 8, 256, 4352, 128, 0.1f, 0, 0, DG_BF16,
                       dummy, sizeof(dummy), nullptr) == DG_EINVAL);          // short workspace
    CHECK(dg_attention(dummy, dummy, dummy, dummy, 16, 8, 256, 4352, 128, 0.1f, 1, 4200,
                       DG_BF16, dummy, sizeof(dummy), nullptr) == DG_EINVAL); // causal beyond keys
    CHECK(dg_attention_noalloc(dummy, dummy, dummy, dummy, 16, 8, 256, 65536, 128, 0.1f, 0, 0,
                               DG_BF16, nullptr) == DG_EINVAL);               // beyond the scratch
    dg_eb_params p = {0.8f, 0.4f, 0.5f, 0.1f, 48};
    CHECK(dg_eb_sample(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 256, 1024,
                       0, &p, 0, 0, nullptr) == DG_EINVAL);
    CHECK(dg_denoise_step_eb(nullptr, nullptr, nullptr, 0, &p, 0, nullptr, nullptr) == DG_EINVAL);
    CHECK(dg_generate_block_eb(nullptr, nullptr, &p, 0, 1, nullptr, nullptr) == DG_EINVAL);
    CHECK(dg_denoise_step_batch(nullptr, nullptr, nullptr, 2, 0, 12, 0, nullptr) == DG_EINVAL);
    CHECK(dg_init_canvas_batch(nullptr, nullptr, nullptr, 2, 0, nullptr) == DG_EINVAL);
    CHECK(dg_generate_block_batch(nullptr, nullptr, 2, 12, 0, nullptr) == DG_EINVAL);
    if (fails) return 1;
    printf("abi driver ok\n");
    return 0;
}
