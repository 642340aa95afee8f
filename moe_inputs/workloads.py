"""Named synthetic workloads of the MoE layer.

Every workload is named by what it is and its sizes.  The K2-shaped ones
take d=7168, E=384, K=8 and scale 2.827 from the Kimi K2 router card
(OpenModelAtlas, "Kimi K2 · Router", the four-step formula and the in/out
shapes); the K3-shaped one takes E=896, K=16, 2 shared experts, latent 3584
and intermediate 3072 from the K3 dimension table of the lilting.ch essay.
The expert width 2048 of the K2 shapes is not printed on the pages: with
3*7168*2048 parameters per expert, 384 routed experts over 60 MoE blocks
come to about 1.0T parameters, which agrees with the "about 1.04T total"
of the llm-arch-kb Kimi K2 entry (section 2, parameter accounting).
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (batch x positions, flattened)
    d: int            # model dimension
    E: int            # routed experts
    K: int            # experts selected per token
    F: int            # routed-expert intermediate size
    n_shared: int     # always-on shared experts
    F_shared: int     # intermediate size of each shared expert
    d_latent: int     # 0: experts act on x; >0: experts act on a d_latent projection of x
    scale: float      # routed scaling factor applied after renormalisation
    act_dtype: str    # "f32" or "bf16": x and the layer output
    w_dtype: str      # "f32" or "bf16": expert, shared and latent weights;
                      # "fp8": routed experts block-scaled FP8, the rest bf16
    bias_range: float  # b ~ U(-bias_range, bias_range)
    zipf_skew: bool   # add a Zipf(1.1)-ranked logit offset (max 0.5) per expert
    router_only: bool  # the workload measures the router alone
    n_group: int = 1   # group-limited choice: expert groups (1: plain top-K)
    topk_group: int = 1  # groups kept per token when n_group > 1
    zipf_scale: float = 0.5  # logit offset of the rank-1 expert when zipf_skew

    @property
    def d_in(self) -> int:
        """Width of the routed experts' input (d, or d_latent in the latent form)."""
        return self.d_latent if self.d_latent else self.d

    @property
    def assignments(self) -> int:
        return self.T * self.K

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=T, name=f"{self.name}@T{T}")


_K2 = dict(d=7168, E=384, K=8, F=2048, n_shared=1, F_shared=2048, d_latent=0,
           scale=2.827, act_dtype="bf16", w_dtype="bf16", bias_range=0.02,
           zipf_skew=True)

WORKLOADS = {
    # fp32 throughout; the oracle finishes in well under a second and all
    # C(32,4) subsets can be enumerated per token.
    "tiny_fp32_t128": Workload(
        name="tiny_fp32_t128", T=128, d=512, E=32, K=4, F=256, n_shared=1,
        F_shared=256, d_latent=0, scale=2.827, act_dtype="f32", w_dtype="f32",
        bias_range=0.01, zipf_skew=False, router_only=False),
    # K2 router alone at 4096 tokens.
    "k2_router_t4096": Workload(name="k2_router_t4096", T=4096,
                                router_only=True, **_K2),
    # The K2 router alone with the group-limited choice of the router card's
    # excerpt at 8 groups of 48 experts, 4 kept (the page's K2 uses one group).
    "k2_router_g8_t4096": Workload(name="k2_router_g8_t4096", T=4096,
                                   router_only=True, n_group=8, topk_group=4, **_K2),
    # K2 layer, decode-sized batch: weight streaming.
    "k2_decode_t256": Workload(name="k2_decode_t256", T=256,
                               router_only=False, **_K2),
    # K2 layer, prefill-sized batch: grouped GEMMs.
    "k2_prefill_t16384": Workload(name="k2_prefill_t16384", T=16384,
                                  router_only=False, **_K2),
    # The K2 prefill layer with a stronger skew: the rank-1 expert's logit
    # offset is 0.8 instead of 0.5, so that the hottest expert of the batch
    # gets about 4x the mean load (0.5 gives 2.25x on this draw: the bias
    # b ~ U(+-0.02) moves a score near the selection threshold by as much as
    # a logit offset of about 0.2, comparable to all but the top offsets).
    "k2_prefill_skew4_t16384": Workload(name="k2_prefill_skew4_t16384", T=16384,
                                        router_only=False, **dict(_K2, zipf_scale=0.8)),
    # The same two K2 layers with the routed experts stored in FP8 with
    # 128 x 128 block scales (the router card's checkpoint note).
    "k2_decode_fp8_t256": Workload(name="k2_decode_fp8_t256", T=256, router_only=False,
                                   **dict(_K2, w_dtype="fp8")),
    "k2_prefill_fp8_t16384": Workload(name="k2_prefill_fp8_t16384", T=16384, router_only=False,
                                      **dict(_K2, w_dtype="fp8")),
    # K3-shaped latent layer.
    "k3_latent_t4096": Workload(
        name="k3_latent_t4096", T=4096, d=7168, E=896, K=16, F=3072,
        n_shared=2, F_shared=3072, d_latent=3584, scale=1.0,
        act_dtype="bf16", w_dtype="bf16", bias_range=0.02, zipf_skew=False,
        router_only=False),
    # Mid-sized bf16 layers for full (every token) parity: several M, N and
    # K tiles and ragged tails, small enough for the oracle to finish in
    # seconds.
    "mid_bf16_t300": Workload(
        name="mid_bf16_t300", T=300, d=1024, E=48, K=6, F=320, n_shared=1,
        F_shared=192, d_latent=0, scale=2.827, act_dtype="bf16",
        w_dtype="bf16", bias_range=0.02, zipf_skew=True, router_only=False),
    "mid_latent_t200": Workload(
        name="mid_latent_t200", T=200, d=768, E=40, K=5, F=192, n_shared=2,
        F_shared=128, d_latent=384, scale=1.0, act_dtype="bf16",
        w_dtype="bf16", bias_range=0.02, zipf_skew=False, router_only=False),
    # FP8 routed experts (128 x 128 scale blocks): d_in and F in whole
    # blocks, several blocks per matrix in both directions.
    "mid_fp8_t300": Workload(
        name="mid_fp8_t300", T=300, d=1024, E=48, K=6, F=384, n_shared=1,
        F_shared=192, d_latent=0, scale=2.827, act_dtype="bf16",
        w_dtype="fp8", bias_range=0.02, zipf_skew=True, router_only=False),
    "mid_fp8_latent_t200": Workload(
        name="mid_fp8_latent_t200", T=200, d=768, E=40, K=5, F=256, n_shared=2,
        F_shared=128, d_latent=384, scale=1.0, act_dtype="bf16",
        w_dtype="fp8", bias_range=0.02, zipf_skew=False, router_only=False),
    "mid_fp32_t77": Workload(
        name="mid_fp32_t77", T=77, d=320, E=20, K=3, F=192, n_shared=0,
        F_shared=0, d_latent=0, scale=2.827, act_dtype="f32", w_dtype="f32",
        bias_range=0.02, zipf_skew=False, router_only=False),
}


def get_workload(name: str) -> Workload:
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    return WORKLOADS[name]
