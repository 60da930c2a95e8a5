"""The Python wrappers reject tensors of the wrong dtype, shape or device before any call into
libdspark.so (which sees bare pointers and would read or write past a short buffer). CPU only:
the library loader is replaced by one that fails the test if it is reached."""
import pytest
import torch

import dspark_markov_draft_amd.binding as B

V, T, BS = 64, 3, 2


@pytest.fixture(autouse=True)
def _no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the C ABI was reached before the argument checks")
    monkeypatch.setattr(B, "lib", forbidden)


def walk_args(**over):
    a = dict(q=torch.zeros(V, 256, dtype=torch.int8), s=torch.zeros(V),
             w1=torch.zeros(V, 256, dtype=torch.bfloat16), base=torch.zeros(BS, T, V),
             start=torch.zeros(BS, dtype=torch.int32), workspace=torch.zeros(4096, dtype=torch.uint8),
             draft_tokens=torch.zeros(BS, T, dtype=torch.int32))
    a.update(over)
    return a


def sample_args(**over):
    a = walk_args(seeds=torch.zeros(BS, dtype=torch.int64), temperature=torch.ones(BS),
                  draft_logits=torch.zeros(BS, T, V, dtype=torch.bfloat16))
    a.update(over)
    return a


BAD_WALK = [
    (dict(base=torch.zeros(BS, T, V, dtype=torch.bfloat16)), "base must be float32"),
    (dict(base=torch.zeros(T, V)), "base must be"),
    (dict(q=torch.zeros(V, 256, dtype=torch.uint8)), "q must be int8"),
    (dict(q=torch.zeros(V - 1, 256, dtype=torch.int8)), "q must have shape"),
    (dict(q=torch.zeros(V, 128, dtype=torch.int8)), "q must have shape"),
    (dict(s=torch.zeros(V, dtype=torch.float64)), "s must be float32"),
    (dict(s=torch.zeros(V + 1)), "s must have shape"),
    (dict(w1=torch.zeros(V, 256, dtype=torch.float64)), "w1 must be"),
    (dict(w1=torch.zeros(V // 2, 256, dtype=torch.bfloat16)), "w1 must have shape"),
    (dict(start=torch.zeros(BS, dtype=torch.int64)), "start must be int32"),
    (dict(start=torch.zeros(BS + 1, dtype=torch.int32)), "start must have shape"),
    (dict(draft_tokens=torch.zeros(BS, T + 1, dtype=torch.int32)), "draft_tokens must have shape"),
    (dict(workspace=torch.zeros(64, 64, dtype=torch.uint8)), "workspace must be"),
    (dict(base=torch.zeros(BS, V, T).transpose(1, 2)), "base must be contiguous"),
]


@pytest.mark.parametrize("over,msg", BAD_WALK)
def test_greedy_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        B.dspark_walk_greedy(**walk_args(**over))


def test_greedy_rejects_bad_logits_buffer():
    with pytest.raises(ValueError, match="out_logits must be float32"):
        B.dspark_walk_greedy(**walk_args(), out_logits=torch.zeros(BS, T, V, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out_logits must have shape"):
        B.dspark_walk_greedy(**walk_args(), out_logits=torch.zeros(BS, T, V - 4))


@pytest.mark.parametrize("over,msg", BAD_WALK + [
    (dict(seeds=torch.zeros(BS, dtype=torch.int32)), "seeds must be int64"),
    (dict(temperature=torch.ones(BS + 1)), "temperature must have shape"),
    (dict(positions=torch.zeros(BS, dtype=torch.int32)), "positions must be int64"),
    (dict(draft_logits=torch.zeros(BS, T, V, dtype=torch.float16)), "draft_logits must be bfloat16"),
    (dict(draft_logits=torch.zeros(BS, T, V - 1, dtype=torch.bfloat16)), "draft_logits must have"),
])
def test_sample_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        B.dspark_walk_sample(**sample_args(**over))


def test_topk_rejects():
    a = walk_args()
    k = 8
    with pytest.raises(ValueError, match="draft_logits must be float32"):
        B.dspark_walk_topk(a["q"], a["s"], a["w1"], a["base"], a["start"], k, a["workspace"],
                           draft_tokens=a["draft_tokens"],
                           draft_logits=torch.zeros(BS, T, V, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="seeds must be int64"):
        B.dspark_walk_topk(a["q"], a["s"], a["w1"], a["base"], a["start"], k, a["workspace"],
                           sample=True, seeds=torch.zeros(BS, dtype=torch.float32),
                           temperature=torch.ones(BS), draft_tokens=a["draft_tokens"])
    with pytest.raises(ValueError, match="q must have shape"):
        B.dspark_walk_topk(torch.zeros(V, 255, dtype=torch.int8), a["s"], a["w1"], a["base"],
                           a["start"], k, a["workspace"], draft_tokens=a["draft_tokens"])


def test_quantize_rejects():
    with pytest.raises(ValueError, match="w2 must be"):
        B.dspark_quantize_w2(torch.zeros(V, 256, dtype=torch.int8))
    with pytest.raises(ValueError, match="w2 must be"):
        B.dspark_quantize_w2(torch.zeros(V * 256))
    with pytest.raises(ValueError, match="q must have shape"):
        B.dspark_quantize_w2(torch.zeros(V, 256), q=torch.zeros(V, 128, dtype=torch.int8))
    with pytest.raises(ValueError, match="s must be float32"):
        B.dspark_quantize_w2(torch.zeros(V, 256), s=torch.zeros(V, dtype=torch.float16))


def test_well_formed_host_tensors_are_rejected_as_not_on_device():
    """Every dtype and shape right, but host memory: still never handed to the library."""
    with pytest.raises(ValueError, match="must be on a CUDA device"):
        B.dspark_walk_greedy(**walk_args())
    with pytest.raises(ValueError, match="must be on a CUDA device"):
        B.dspark_walk_sample(**sample_args())
    with pytest.raises(ValueError, match="must be on a CUDA device"):
        B.dspark_quantize_w2(torch.zeros(V, 256))
