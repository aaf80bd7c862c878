"""Random parity sweep against the oracle for as long as asked (needs an MI355X):

    python tests/fuzz_parity.py SEED SECONDS

draws prefill (MHA and GQA with groups up to 8, causal with N <= M or not,
head dims 32-256, fp16 and bf16, N and M up to a few hundred), FP8 Q/K
prefill, decode (chunks of 128-2048 keys, the two-launch and the one-launch
paths), FP8-KV decode and paged decode (page sizes 16-256, both cache
layouts) shapes from the seed, compares each
with the oracle at the fixed tolerances (V scaled by 0.25, as in
test_parity_random.py) and exits non-zero if any case misses them.  Not
collected by pytest (a time-bounded stress run, not a fixed test).
"""
import sys, time
import pathlib
ROOT = pathlib.Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT)); sys.path.insert(0, str(ROOT / 'tests'))
import numpy as np, torch, oracle
from workloads import prefill_inputs, decode_inputs, prefill_fp8qk_inputs
from tests.test_parity_gpu import paged_inputs
import attention_attn_fwd_06_amd as A
DEV = "cuda"; TOL_O = {"f16": 2e-3, "bf16": 8e-3}; TOL_L = 1e-3
f64 = lambda t: t.detach().float().cpu().double().numpy()
me = lambda a, b: float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0
rng = np.random.default_rng(int(sys.argv[1]) if len(sys.argv) > 1 else 7)
budget = float(sys.argv[2]) if len(sys.argv) > 2 else 240
t0 = time.time(); n = 0; bad = []
while time.time() - t0 < budget:
    kind = rng.choice(["prefill", "prefill", "decode", "paged", "fp8qk", "fp8kv"])
    dt = str(rng.choice(["f16", "bf16"])); d = int(rng.choice([32, 64, 128, 256]))
    try:
        if kind == "prefill":
            Hkv = int(rng.choice([1, 2, 3, 4])); g = int(rng.choice([1, 2, 3, 4, 5, 8])); B = int(rng.integers(1, 3))
            causal = bool(rng.integers(0, 2)); N = int(rng.integers(1, 300)); M = int(rng.integers(N if causal else 1, 520))
            case = (kind, B, N, M, Hkv * g, Hkv, d, dt, causal); print(case, flush=True)
            q, k, v = prefill_inputs(B, Hkv * g, Hkv, N, M, d, dt, seed=n); v = v * 0.25
            sc = float(np.float32(d ** -0.5))
            o, l = A.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=sc); torch.cuda.synchronize()
            Or, Lr = oracle.attn_ref(q, k, v, sc, causal); eo, el = me(f64(o), Or), me(f64(l), Lr)
        elif kind == "decode":
            Hkv = int(rng.choice([1, 2, 4, 8])); g = int(rng.choice([1, 2, 3, 4, 8, 16])); B = int(rng.integers(1, 3))
            M = int(rng.integers(1, 5000)); chunk = int(rng.choice([128, 256, 512, 1024, 2048]))
            case = (kind, B, Hkv * g, Hkv, M, d, dt, chunk); print(case, flush=True)
            q, k, v = decode_inputs(B, Hkv * g, Hkv, M, d, dt, seed=n); v = v * 0.25
            sc = float(np.float32(d ** -0.5))
            o, l, _, _ = A.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), chunk, sc)
            of, lf = A.attn_decode_fused(q.to(DEV), k.to(DEV), v.to(DEV), sc); torch.cuda.synchronize()
            Or, Lr, _, _ = oracle.decode_ref(q, k, v, sc, chunk)
            eo = max(me(f64(o), Or), me(f64(of), Or)); el = max(me(f64(l), Lr), me(f64(lf), Lr))
        elif kind == "fp8qk":
            d = int(rng.choice([64, 128]))
            Hkv = int(rng.choice([1, 2, 4])); g = int(rng.choice([1, 2, 4])); B = int(rng.integers(1, 3))
            causal = bool(rng.integers(0, 2)); N = int(rng.integers(1, 300)); M = int(rng.integers(N if causal else 1, 520))
            case = (kind, B, N, M, Hkv * g, Hkv, d, dt, causal); print(case, flush=True)
            q8, k8, v, qs, ks = prefill_fp8qk_inputs(B, Hkv * g, Hkv, N, M, d, dt, seed=n); v = v * 0.25
            sc = float(np.float32(d ** -0.5))
            o, l = A.attn_fwd_fp8qk(q8.to(DEV), k8.to(DEV), v.to(DEV), qs, ks, causal=causal, scale=sc)
            torch.cuda.synchronize()
            Or, Lr = oracle.attn_fp8qk_ref(q8.numpy(), k8.numpy(), v, qs, ks, sc, causal)
            eo, el = me(f64(o), Or), me(f64(l), Lr)
        elif kind == "fp8kv":
            d = int(rng.choice([32, 64, 128]))
            Hkv = int(rng.choice([1, 2, 4, 8])); g = int(rng.choice([1, 2, 4, 8])); B = int(rng.integers(1, 3))
            M = int(rng.integers(1, 5000)); chunk = int(rng.choice([128, 256, 512, 1024]))
            case = (kind, B, Hkv * g, Hkv, M, d, dt, chunk); print(case, flush=True)
            q, k, v = decode_inputs(B, Hkv * g, Hkv, M, d, dt, seed=n); v = v * 0.25
            ks = float(np.float32(float(k.float().abs().max()) / 448.0)); vs = float(np.float32(float(v.float().abs().max()) / 448.0))
            kc = (k.float() / ks).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
            vc = (v.float() / vs).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
            sc = float(np.float32(d ** -0.5))
            o, l, _, _ = A.attn_decode_fp8kv(q.to(DEV), kc.to(DEV), vc.to(DEV), ks, vs, chunk, sc)
            of, lf = A.attn_decode_fp8kv_fused(q.to(DEV), kc.to(DEV), vc.to(DEV), ks, vs, sc); torch.cuda.synchronize()
            Or, Lr, _, _ = oracle.decode_fp8kv_ref(q, kc.numpy(), vc.numpy(), ks, vs, sc, chunk)
            eo = max(me(f64(o), Or), me(f64(of), Or)); el = max(me(f64(l), Lr), me(f64(lf), Lr))
        else:
            Hkv = int(rng.choice([1, 2, 4])); g = int(rng.choice([1, 2, 4, 8])); B = int(rng.integers(1, 4))
            lens = [int(x) for x in rng.integers(1, 3000, size=B)]; bs = int(rng.choice([16, 32, 48, 64, 112, 256]))
            hm = bool(rng.integers(0, 2)); chunk = int(rng.choice([128, 256, 512]))
            case = (kind, B, Hkv * g, Hkv, tuple(lens), d, dt, bs, hm, chunk); print(case, flush=True)
            q, kc, vc, kv_k, kv_v, table, sl = paged_inputs(B, Hkv * g, Hkv, lens, d, dt, bs, seed=n, head_major=hm)
            vc.mul_(0.25)
            view = (lambda t: t.transpose(1, 2)) if hm else (lambda t: t)
            sc = float(np.float32(d ** -0.5))
            kd, vd = view(kc.to(DEV)), view(vc.to(DEV))
            o, l, _, _ = A.attn_decode_paged(q.to(DEV), kd, vd, table.to(DEV), sl.to(DEV), chunk, sc)
            of, lf = A.attn_decode_paged_fused(q.to(DEV), kd, vd, table.to(DEV), sl.to(DEV), sc); torch.cuda.synchronize()
            Or, Lr, _, _ = oracle.paged_decode_ref(q, kv_k, kv_v, table.clamp(min=0), sl, sc, chunk)
            eo = max(me(f64(o), Or), me(f64(of), Or)); el = max(me(f64(l), Lr), me(f64(lf), Lr))
    except Exception as e:
        print("ERROR", case, repr(e)[:300], flush=True); bad.append((case, 'error')); n += 1; continue
    if not (eo <= TOL_O[dt] and el <= TOL_L):
        print("FAIL", case, eo, el, flush=True); bad.append((case, eo, el))
    n += 1
print(f"cases {n}, failures {len(bad)}", flush=True)
for b in bad: print(b)
sys.exit(1 if bad else 0)
